"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer and byte results (dequantised bf16 weights, routing indices, counts,
offsets, permutations) must match bit for bit. Floating-point outputs must lie
within 1e-2 * rms(ref) of the float64 reference plus half a bf16 ulp of the
reference (the final bf16 rounding of the output), and their rms error must
stay below 3e-3 * rms(ref). Router logits must lie within the fp32 summation
bound; the selected expert sets must then agree wherever the oracle's top-k
boundary gap is wider than twice that bound.
"""
import numpy as np
import pytest

import oracle as O
from workloads import get_workload, gen_all, gen_logits, gen_expert, gen_x, gen_router
from workloads.configs import Dims, Workload

from lmoe_testutil import (log, to_dev, upload, alloc_routing, run_forward, check_out,
                           logits_bound, check_routing_against_oracle, check_routing_exact,
                           flip_allowance_fn)
from lmoe_layer_checks import full_small as _full_small, full_size as _full_size, \
    every_token_isolated as _every_token_isolated

pytestmark = pytest.mark.gpu


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


# ----------------------------------------------------------------------------
# Dequantisation
# ----------------------------------------------------------------------------

def _dequant_gpu(lm, dev, q, s, rows, K):
    import torch
    out = torch.empty((rows, K), dtype=torch.int16, device=dev)
    lm.debug_dequant_mxfp4(to_dev(q, dev), to_dev(s, dev), rows, K, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def _compare_dequant(got, ref64):
    ref = O.bf16_from_f64(ref64)
    nan = np.isnan(ref64)
    got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert np.array_equal(nan, got_nan), "NaN placement differs"
    mism = np.nonzero((got != ref) & ~nan)
    assert mism[0].size == 0, (
        f"{mism[0].size} mismatches, first {tuple(m[0] for m in mism)}: "
        f"got {hex(got[mism][0])} want {hex(ref[mism][0])}")


def test_dequant_exhaustive_codes_and_exponents(lm, dev):
    log("dequant: 16 codes x 256 exponents")
    N, K = 256, 64
    codes = np.tile(np.arange(K) % 16, (N, 1)).astype(np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = np.stack([np.arange(256), (np.arange(256) + 97) % 256], axis=1).astype(np.uint8)
    got = _dequant_gpu(lm, dev, q, s, N, K)
    _compare_dequant(got, O.dequant_mxfp4(q, s, N, K))


def test_dequant_k3_expert_matrix(lm, dev):
    log("dequant: one K3 gate matrix (2048 x 3584) and one down matrix")
    w = get_workload("decode")
    ex = gen_expert(w, 5)
    for qk, sk, N, K in (("gate_q", "gate_s", 2048, 3584), ("down_q", "down_s", 3584, 2048)):
        got = _dequant_gpu(lm, dev, ex[qk], ex[sk], N, K)
        _compare_dequant(got, O.dequant_mxfp4(ex[qk], ex[sk], N, K))


# ----------------------------------------------------------------------------
# Routing on given logits: bit-exact
# ----------------------------------------------------------------------------

def _route_given(lm, dev, logits: np.ndarray, k: int):
    import torch
    T, E = logits.shape
    d = Dims(T=T, L=32, E=E, k=k, I=32, S=0, Is=0)
    r = alloc_routing(d, dev)
    r["logits"] = to_dev(logits.astype(np.float32), dev)
    ws = torch.zeros(max(1, lm.workspace_bytes(d)), dtype=torch.uint8, device=dev)
    lm.route(d, None, None, True, r, ws)
    torch.cuda.synchronize()
    return {kk: v.cpu().numpy() for kk, v in r.items()}


def _check_route_exact(res, logits, k, what):
    check_routing_exact(res, logits, k, what)


@pytest.mark.parametrize("E,k", [(8, 1), (8, 8), (40, 16), (33, 5), (1024, 32), (896, 16)])
def test_topk_edge_values(lm, dev, E, k):
    rng = np.random.default_rng(E * 7 + k)
    pool = np.array([1.5, 1.5, 0.0, -0.0, -2.0, 3.0, np.nan, -np.inf, np.inf, 0.25], np.float32)
    T = 70
    lg = rng.choice(pool, size=(T, E)).astype(np.float32)
    lg[:30] = rng.normal(size=(30, E)).astype(np.float32)
    lg[30:40] = 0.0                       # every logit tied
    res = _route_given(lm, dev, lg, k)
    _check_route_exact(res, lg, k, f"edge values E={E} k={k}")


@pytest.mark.parametrize("name", ["tiny", "ragged_skew"])
def test_route_given_logits_small(lm, dev, name):
    w = get_workload(name)
    lg = gen_logits(Workload(name, w.seed, w.dims, logits_given=True, tie_group=min(12, w.dims.E)))
    res = _route_given(lm, dev, lg, w.dims.k)
    _check_route_exact(res, lg, w.dims.k, name)


def test_route_given_logits_skewed_full(lm, dev):
    w = get_workload("skewed")
    log("skewed: generating 8192 x 896 logits")
    lg = gen_logits(w)
    res = _route_given(lm, dev, lg, w.dims.k)
    _check_route_exact(res, lg, w.dims.k, "skewed T=8192")


# ----------------------------------------------------------------------------
# Whole layer on small shapes: every token
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ragged", "ragged_prefill", "ragged_skew"])
def test_forward_small_workloads(lm, dev, name):
    _full_small(lm, dev, get_workload(name))


@pytest.mark.parametrize("T", [1, 2, 3, 31, 33, 64, 65, 255, 700])
def test_forward_token_counts(lm, dev, T):
    """Both tile paths, partial row tiles and single-token decode."""
    _full_small(lm, dev, get_workload("tiny").with_T(T))


@pytest.mark.parametrize("T", [16, 160, 400])
def test_forward_whole_exponent_windows(lm, dev, T):
    """Widths whose rows hold whole 16-block exponent windows (L/32 and I/32
    multiples of 16, as on the Kimi-K3 layer), on which the grouped kernels
    read exponents through LDS (large tiles) or hold a wave's K range of them
    in registers (small tiles, 16 tokens); at 400 tokens over 8 experts groups
    exceed 96 rows."""
    _full_small(lm, dev, Workload(f"windows{T}", 26, Dims(T=T, L=1024, E=8, k=2, I=512, S=1,
                                                           Is=256)))


@pytest.mark.parametrize("variant", ["k1", "kE", "noshared", "Is_ne_I", "wide_scales"])
def test_forward_degenerate_cases(lm, dev, variant):
    base = get_workload("ragged")
    d = base.dims
    if variant == "k1":
        w = Workload("k1", 21, Dims(T=50, L=d.L, E=d.E, k=1, I=d.I, S=2, Is=d.Is))
    elif variant == "kE":
        w = Workload("kE", 22, Dims(T=20, L=160, E=12, k=12, I=96, S=1, Is=64))
    elif variant == "noshared":
        w = Workload("noshared", 23, Dims(T=40, L=d.L, E=d.E, k=d.k, I=d.I, S=0, Is=0))
    elif variant == "Is_ne_I":
        w = Workload("Is_ne_I", 24, Dims(T=90, L=288, E=20, k=4, I=64, S=3, Is=416))
    else:
        w = Workload("wide_scales", 25, Dims(T=30, L=256, E=16, k=4, I=128, S=1, Is=128),
                     scales=("uniform", 100, 140))
    _full_small(lm, dev, w)


def test_forward_deterministic(lm, dev):
    w = get_workload("ragged_prefill")
    inp = gen_all(w)
    dinp = upload(inp, dev)
    a, _ = run_forward(lm, w, dinp)
    b, _ = run_forward(lm, w, dinp)
    assert np.array_equal(a, b)


def test_forward_without_routing_outputs(lm, dev):
    import torch
    w = get_workload("tiny")
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    ref, _ = run_forward(lm, w, dinp)
    out = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.forward(d, dinp["x"], dinp, False, None, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), ref)


def test_zero_tokens_is_noop(lm, dev):
    import torch
    w = get_workload("tiny")
    inp = gen_all(w)
    dinp = upload(inp, dev)
    d = Dims(T=0, L=w.dims.L, E=w.dims.E, k=w.dims.k, I=w.dims.I, S=w.dims.S, Is=w.dims.Is)
    out = torch.zeros((1, d.L), dtype=torch.int16, device=dev)
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    lm.forward(d, dinp["x"], dinp, False, None, out, ws)
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0


# ----------------------------------------------------------------------------
# Full K3-sized workloads. Routing on every token: with given logits the
# oracle's selection, weights and grouping must match bit for bit (weights
# within the derived softmax bound); with computed logits the GPU logits must
# lie within the fp32 summation bound of the oracle's, the oracle's selection
# and grouping applied to the GPU's own logits must match bit for bit, and the
# selected sets must agree wherever the boundary gap is clear. Outputs: on
# sampled tokens with the workload's real experts, and on every token with all
# but a few experts silenced (below).
# ----------------------------------------------------------------------------

def test_full_decode(lm, dev):
    _full_size(lm, dev, get_workload("decode"), 1)


def test_full_decode_three_tokens(lm, dev):
    """Three K3 decode tokens in one call (seed 1's inputs) on the fused
    multi-token kernel. Every token is checked."""
    w = get_workload("decode").with_T(3, "decode_t3")
    assert lm.path_name(w.dims) == "fused_multi"
    _full_size(lm, dev, w, 3)


def test_full_batched_decode(lm, dev):
    _full_size(lm, dev, get_workload("batched_decode"), 3)


def test_full_prefill(lm, dev):
    _full_size(lm, dev, get_workload("prefill"), 3)


def test_full_skewed(lm, dev):
    _full_size(lm, dev, get_workload("skewed"), 3)


def test_full_decode_i3072(lm, dev):
    """The expert width implied by the pages' per-expert size."""
    _full_size(lm, dev, get_workload("decode_i3072"), 1)


def test_full_prefill_i3072(lm, dev):
    _full_size(lm, dev, get_workload("prefill_i3072"), 3)


def test_full_decode_tp8(lm, dev):
    """One GPU's eighth of every expert (I = Is = 256), router whole."""
    _full_size(lm, dev, get_workload("decode_tp8"), 1)


# ----------------------------------------------------------------------------
# Every token at full size. The workload runs with its real router, routing and
# shapes, but every expert outside a kept set has all gate codes zero, so its
# routes give h = bf16(silu(0) u) = 0 and y = 0: each output is then the kept
# experts' weighted partials plus the shared experts, which the oracle computes
# for all T tokens at the cost of the kept experts alone. Kept: the hottest
# expert (every one of its tokens checked, over all of its row tiles), the
# coldest non-empty one, and one whose group just passes a 96-row tile.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["prefill", "skewed", "batched_decode"])
def test_full_every_token_isolated(lm, dev, name):
    _every_token_isolated(lm, dev, get_workload(name))


# ----------------------------------------------------------------------------
# The Kimi-K3 widths (L = 3584, I = Is = 2048, k = 16) with few experts, so the
# oracle runs the whole layer on every token: computed logits with 2-4 row
# tiles per group, and given Zipf-skewed logits with groups of 1 to 16 row
# tiles. Both use the whole-exponent-row path of the grouped kernels.
# ----------------------------------------------------------------------------

K3W = dict(L=3584, k=16, I=2048, S=2, Is=2048)


@pytest.mark.parametrize("w", [
    Workload("k3w_e64_t1024", 31, Dims(T=1024, E=64, **K3W)),
    Workload("k3w_e48_t1536_skew", 32, Dims(T=1536, E=48, **K3W), logits_given=True),
], ids=lambda w: w.name)
def test_k3_width_every_token(lm, dev, w):
    _full_small(lm, dev, w)


# ----------------------------------------------------------------------------
# The shared experts on the library's second stream (untraced grouped calls)
# against the same layer with every stage on the caller's stream (traced)
# ----------------------------------------------------------------------------

def _hip_events(n):
    import ctypes
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert lib.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    return evs


@pytest.mark.parametrize("name", ["ragged", "ragged_prefill", "ragged_skew"])
def test_side_stream_matches_single_stream(lm, dev, name):
    import torch
    w = get_workload(name)
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    r = {"logits": dinp["logits"]} if w.logits_given else None
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    side = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    lm.forward(d, dinp["x"], dinp, w.logits_given, r, side, ws)
    one = torch.empty_like(side)
    lm.forward_traced(d, dinp["x"], dinp, w.logits_given, r, one, ws,
                      _hip_events(lm.NUM_STAGE_EVENTS))
    torch.cuda.synchronize()
    assert np.array_equal(side.cpu().numpy(), one.cpu().numpy())


@pytest.mark.parametrize("name", ["ragged_prefill", "ragged_skew"])
def test_forward_ex_side_stream_choices(lm, dev, name):
    """lmoe_forward_ex with the shared experts on a caller stream forked and
    joined by caller events, and with every stage on one stream: both equal
    lmoe_forward bit for bit."""
    import torch
    w = get_workload(name)
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    r = {"logits": dinp["logits"]} if w.logits_given else None
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    ref = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    lm.forward(d, dinp["x"], dinp, w.logits_given, r, ref, ws)
    side = torch.cuda.Stream()
    fork, join = _hip_events(2)
    for use_side in (True, False, True):
        out = torch.empty_like(ref)
        if use_side:
            lm.forward_ex(d, dinp["x"], dinp, w.logits_given, r, out, ws, side.cuda_stream,
                          fork, join)
        else:
            lm.forward_ex(d, dinp["x"], dinp, w.logits_given, r, out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy()), f"side={use_side}"


def test_back_to_back_calls_reuse_workspace(lm, dev):
    """Two calls on one stream and one workspace with no wait between them:
    the second call's shared experts must not start before the first call is
    done with the workspace."""
    import torch
    w = get_workload("ragged_prefill")
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    x2 = torch.flip(dinp["x"], dims=[0]).contiguous()
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    ref = []
    for x in (dinp["x"], x2):
        o = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
        lm.forward(d, x, dinp, False, None, o, ws)
        torch.cuda.synchronize()
        ref.append(o.cpu().numpy())
    outs = [torch.empty((d.T, d.L), dtype=torch.int16, device=dev) for _ in range(4)]
    for i, o in enumerate(outs):
        lm.forward(d, dinp["x"] if i % 2 == 0 else x2, dinp, False, None, o, ws)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert np.array_equal(o.cpu().numpy(), ref[i % 2]), f"call {i}"


@pytest.mark.parametrize("name", ["ragged", "ragged_prefill", "tiny1"])
def test_graph_capture_replays_match_eager(lm, dev, name):
    """lmoe_forward captured into a HIP graph (the grouped path forks the
    shared experts onto the library's second stream inside the capture; the
    single-token path is one persistent kernel): several replays, with eager
    calls in between, each equal to the eager output."""
    import torch
    if name == "tiny1":
        w = Workload("tiny1", 40, Dims(T=1, L=256, E=32, k=4, I=128, S=2, Is=128),
                     scales=("uniform", 120, 130))
    else:
        w = get_workload(name)
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    ref = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    lm.forward(d, dinp["x"], dinp, False, None, ref, ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lm.forward(d, dinp["x"], dinp, False, None, out, ws)
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy()), f"replay {i}"
        eager = torch.empty_like(ref)
        lm.forward(d, dinp["x"], dinp, False, None, eager, ws)
        torch.cuda.synchronize()
        assert np.array_equal(eager.cpu().numpy(), ref.cpu().numpy()), f"eager after replay {i}"

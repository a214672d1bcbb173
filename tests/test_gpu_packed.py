"""GPU parity of the tile-packed path: lmoe_pack_weights against the layout
include/lmoe.h states (bit for bit), and lmoe_forward_packed against the
float64 oracle with the same checks as the row-major path."""
import numpy as np
import pytest

from workloads import get_workload, gen_all
from workloads.configs import Dims, Workload

from lmoe_testutil import log, upload, pack_on_device
from lmoe_layer_checks import full_small, full_size, every_token_isolated

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
# The packed layout, restated from the header's description in numpy
# ----------------------------------------------------------------------------

def _gu_rows(gate, up):
    """[E][I][X] gate and up -> [E][2I][X] in packed row order: tile n holds
    gate rows 16n..16n+15, then up rows 16n..16n+15."""
    E, I, X = gate.shape
    g = gate.reshape(E, I // 16, 16, X)
    u = up.reshape(E, I // 16, 16, X)
    return np.concatenate([g, u], axis=2).reshape(E, 2 * I, X)


def _pack_codes(q, N, K):
    """q [E][N][K/2] -> codes [E][N32][K128][2][64][16]: lane l = 32h + r,
    half j: row 32n + r, block 4c + 2h + j."""
    E = q.shape[0]
    N32, K128, nblk = -(-N // 32), -(-K // 128), K // 32
    pad = np.zeros((E, N32 * 32, K128 * 4, 16), np.uint8)
    pad[:, :N, :nblk] = q.reshape(E, N, nblk, 16)
    t = pad.reshape(E, N32, 32, K128, 2, 2, 16)        # e n r c h j b
    return t.transpose(0, 1, 3, 5, 4, 2, 6).reshape(-1)


def _pack_scales(s, N, K):
    """s [E][N][K/32] -> exponents [E][N32][K512][64][8]: lane l = 32h + r,
    byte b = 2q + j: row 32n + r, block 4(4w + q) + 2h + j; 127 past the end."""
    E = s.shape[0]
    N32, K512, nblk = -(-N // 32), -(-K // 512), K // 32
    pad = np.full((E, N32 * 32, K512 * 16), 127, np.uint8)
    pad[:, :N, :nblk] = s.reshape(E, N, nblk)
    t = pad.reshape(E, N32, 32, K512, 4, 2, 2)          # e n r w q h j
    return t.transpose(0, 1, 3, 5, 2, 4, 6).reshape(-1)


@pytest.mark.parametrize("w", [
    get_workload("tiny"),
    get_workload("ragged"),                               # rows and K past the tiles
    Workload("k3w_e2", 33, Dims(T=1, L=3584, E=2, k=1, I=2048, S=0, Is=0)),
], ids=lambda w: w.name)
def test_pack_layout_matches_header(lm, dev, w):
    import torch
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    pk = pack_on_device(lm, d, dinp)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in pk.items()}
    want = {
        "gu_q": _pack_codes(_gu_rows(inp["gate_q"], inp["up_q"]), 2 * d.I, d.L),
        "gu_s": _pack_scales(_gu_rows(inp["gate_s"], inp["up_s"]), 2 * d.I, d.L),
        "down_q": _pack_codes(inp["down_q"], d.L, d.I),
        "down_s": _pack_scales(inp["down_s"], d.L, d.I),
    }
    for k in want:
        assert got[k].size == want[k].size, k
        bad = np.nonzero(got[k] != want[k])[0]
        assert bad.size == 0, f"{k}: {bad.size} bytes differ, first at {bad[0]}"
    log(f"{w.name}: packed layout bit-exact ({sum(v.size for v in want.values())} bytes)")


# ----------------------------------------------------------------------------
# lmoe_forward_packed against the oracle
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ragged", "ragged_prefill", "ragged_skew"])
def test_packed_small_workloads(lm, dev, name):
    full_small(lm, dev, get_workload(name), packed=True)


@pytest.mark.parametrize("T", [1, 2, 31, 33, 129, 257, 700])
def test_packed_token_counts(lm, dev, T):
    """Row tiles of 1-4 MFMA tiles, groups past 128 routes, single tokens."""
    full_small(lm, dev, get_workload("tiny").with_T(T), packed=True)


@pytest.mark.parametrize("variant", ["k1", "kE", "noshared", "Is_ne_I", "wide_scales",
                                     "odd_width"])
def test_packed_degenerate_cases(lm, dev, variant):
    d = get_workload("ragged").dims
    w = {
        "k1": Workload("k1", 21, Dims(T=50, L=d.L, E=d.E, k=1, I=d.I, S=2, Is=d.Is)),
        "kE": Workload("kE", 22, Dims(T=20, L=160, E=12, k=12, I=96, S=1, Is=64)),
        "noshared": Workload("noshared", 23, Dims(T=40, L=d.L, E=d.E, k=d.k, I=d.I, S=0, Is=0)),
        "Is_ne_I": Workload("Is_ne_I", 24, Dims(T=90, L=288, E=20, k=4, I=64, S=3, Is=416)),
        "wide_scales": Workload("wide_scales", 25, Dims(T=30, L=256, E=16, k=4, I=128, S=1,
                                                        Is=128), scales=("uniform", 100, 140)),
        # I = 32 (one packed gate/up tile half empty), L not a multiple of 128
        "odd_width": Workload("odd_width", 27, Dims(T=70, L=96, E=10, k=3, I=32, S=1, Is=32)),
    }[variant]
    full_small(lm, dev, w, packed=True)


K3W = dict(L=3584, k=16, I=2048, S=2, Is=2048)


@pytest.mark.parametrize("w", [
    Workload("k3w_e64_t1024", 31, Dims(T=1024, E=64, **K3W)),
    Workload("k3w_e48_t1536_skew", 32, Dims(T=1536, E=48, **K3W), logits_given=True),
], ids=lambda w: w.name)
def test_packed_k3_width_every_token(lm, dev, w):
    full_small(lm, dev, w, packed=True)


def test_packed_full_prefill(lm, dev):
    full_size(lm, dev, get_workload("prefill"), 3, packed=True)


@pytest.mark.parametrize("name", ["prefill", "skewed", "batched_decode"])
def test_packed_full_every_token_isolated(lm, dev, name):
    every_token_isolated(lm, dev, get_workload(name), packed=True)


def test_packed_side_stream_choices(lm, dev):
    """The shared experts on a caller stream or on the call's stream: the
    same bits."""
    import torch
    from test_gpu_parity import _hip_events
    w = get_workload("ragged_prefill")
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    pk = pack_on_device(lm, d, dinp)
    wts = {**dinp, **pk}
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    ref = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    lm.forward_packed(d, dinp["x"], wts, False, None, ref, ws)
    side = torch.cuda.Stream()
    fork, join = _hip_events(2)
    for use_side in (True, False):
        out = torch.empty_like(ref)
        if use_side:
            lm.forward_packed(d, dinp["x"], wts, False, None, out, ws, side.cuda_stream, fork,
                              join)
        else:
            lm.forward_packed(d, dinp["x"], wts, False, None, out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy()), f"side={use_side}"

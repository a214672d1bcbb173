"""GPU parity of the quantised-activation path (lmoe_exec.act_format on
tile-packed experts): the routed GEMMs' inputs quantised to FP8 E4M3 or FP4
E2M1 with one E8M0 scale per 32 values and multiplied with the MXFP4 weights
on the scaled MFMA, against the oracle's statement of the same quantisation
(TokenSpeed's precision table, row "Routed-expert GEMMs"; the scale reading
in oracle/lmoe_oracle.py).

The quantiser itself must match the oracle bit for bit (codes and exponent
bytes: the same power-of-two scaling is exact, and the rounding is an integer
decision both sides take on the same value). The layer must match the oracle
on every token within the output bound, plus the h-rounding allowance where
that alone fails (a flipped bf16 h can move its quantised value by one grid
step)."""
import numpy as np
import pytest

import oracle as O
from workloads import get_workload
from workloads.configs import Dims, Workload

from lmoe_testutil import log
from lmoe_layer_checks import full_small, every_token_isolated

pytestmark = pytest.mark.gpu

FORMATS = {"e4m3": 1, "e2m1": 2}


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


def _special_rows(fmt: str, K: int, rng) -> np.ndarray:
    """Rows (float64 values, exactly bf16) that exercise the rounding: every
    midpoint of the element grid under several block scales, negative zero,
    zero blocks, blocks that saturate, tiny (bf16 subnormal) blocks."""
    mags = np.unique(np.abs(O.format_values(np.arange(16 if fmt == "e2m1" else 127), fmt)))
    mids = (mags[:-1] + mags[1:]) / 2
    top = mags[-1]
    emax = O.ACT_EMAX[fmt]
    rows = []
    for X in (-3, 0, 5):
        vals = np.concatenate([mids, -mids, mags, -mags])
        for i in range(0, vals.size, 31):
            blk = np.zeros(32)
            part = vals[i:i + 31]
            blk[:part.size] = part
            blk[31] = 2.0 ** emax * 1.5          # the block maximum: fixes X
            rows.append(blk * 2.0 ** X)
    sat = np.full(32, 2.0 ** (emax + 1) * 0.99)  # rounds above the largest value
    sat[1::2] *= -1
    rows.append(sat)
    rows.append(np.zeros(32))
    rows.append(np.full(32, -0.0))
    rows.append(np.ldexp(rng.integers(1, 128, 32).astype(float), -133))  # bf16 subnormals
    rows.append(rng.normal(size=32) * 2.0 ** -120)
    flat = np.concatenate(rows)
    flat = np.concatenate([flat, np.zeros((-flat.size) % K)])
    return O.bf16_from_f64(flat.reshape(-1, K))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantize_hook_bit_exact(lm, dev, fmt):
    import torch
    rng = np.random.default_rng(11)
    K = 256
    rand = O.bf16_from_f64(rng.normal(size=(300, K)) *
                           np.ldexp(1.0, rng.integers(-30, 30, size=(300, 1))))
    bits = np.concatenate([_special_rows(fmt, K, rng), rand])
    rows = bits.shape[0]
    src = torch.from_numpy(bits.view(np.int16).copy()).to(dev)
    nbytes = K if fmt == "e4m3" else K // 2
    codes = torch.zeros((rows, nbytes), dtype=torch.uint8, device=dev)
    exps = torch.zeros((rows, K // 32), dtype=torch.uint8, device=dev)
    lm.debug_quantize_act(src, rows, K, FORMATS[fmt], codes, exps)
    torch.cuda.synchronize()
    got_c, got_e = codes.cpu().numpy(), exps.cpu().numpy()
    want_c, want_e = O.mx_quantize(O.f64_from_bf16(bits), fmt)
    assert np.array_equal(got_e, want_e), f"{fmt}: exponents differ at {np.argwhere(got_e != want_e)[:4]}"
    if fmt == "e2m1":
        got_c = np.stack([got_c & 15, got_c >> 4], axis=-1).reshape(rows, K)
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, (f"{fmt}: codes differ at {bad[:4].tolist()}: got "
                           f"{got_c[tuple(bad[0])]} want {want_c[tuple(bad[0])]}")
    log(f"quantiser {fmt}: {rows} x {K} bit-exact")


SMALL = [
    Workload("q_tiny", 60, Dims(T=8, L=256, E=32, k=4, I=128, S=2, Is=128),
             scales=("uniform", 120, 130)),
    Workload("q_ragged", 61, Dims(T=301, L=384, E=40, k=5, I=640, S=1, Is=160),
             scales=("uniform", 118, 132)),
    # K3 widths, few experts: groups over several 96-row tiles
    Workload("q_k3w", 62, Dims(T=1200, L=3584, E=48, k=4, I=2048, S=2, Is=2048)),
    Workload("q_noshared", 63, Dims(T=33, L=256, E=16, k=1, I=256, S=0, Is=0),
             scales=("uniform", 118, 132)),
    # K a multiple of 256 (the MXFP4 pair-copy kernel) with 6 and 4 chunks:
    # a ring group of four left half full, and groups of 1-3 row tiles
    Workload("q_pairs", 65, Dims(T=400, L=768, E=12, k=3, I=512, S=1, Is=256),
             scales=("uniform", 118, 132)),
    # the same kernel with about 50 routes an expert: mostly two 32-row MFMA
    # tiles a group (K = 512 and 256: 4 and 2 chunks)
    Workload("q_pairs_mt2", 66, Dims(T=300, L=512, E=24, k=4, I=256, S=1, Is=256),
             scales=("uniform", 118, 132)),
]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_packed_quantised_small(lm, dev, w, fmt):
    full_small(lm, dev, w, packed=True, act=fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("T", [1, 2, 129, 700])
def test_packed_quantised_token_counts(lm, dev, T, fmt):
    w = Workload(f"q_t{T}", 64, Dims(T=T, L=256, E=32, k=4, I=128, S=2, Is=128),
                 scales=("uniform", 120, 130))
    full_small(lm, dev, w, packed=True, act=fmt)


def test_packed_quantised_prefill_every_token_isolated(lm, dev):
    """The K3 prefill chunk with MXFP4 activations, the pages' prefill
    precision: every token, all but a few experts silenced."""
    every_token_isolated(lm, dev, get_workload("prefill"), packed=True, act="e2m1")


def test_packed_quantised_batched_decode_every_token_isolated(lm, dev):
    """K3 batched decode (T=64) with FP8 activations, the pages' small-decode
    precision: every token, all but a few experts silenced."""
    every_token_isolated(lm, dev, get_workload("batched_decode"), packed=True, act="e4m3")

"""lmoe_forward_noalloc (the workspace in the library's static per-GPU
scratch) against lmoe_forward on a caller workspace: outputs and routing
bit for bit, over consecutive calls on the shared scratch, each later call
on a smaller input than the one before."""
import numpy as np
import pytest

from workloads import gen_all, gen_x, get_workload
from workloads.configs import Dims, Workload

from lmoe_testutil import log, upload, alloc_routing

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


def _both(lm, dev, w: Workload, dinp, x):
    """(out, routing) of lmoe_forward and of lmoe_forward_noalloc on x."""
    import torch
    d = w.dims
    res = []
    for noalloc in (False, True):
        r = alloc_routing(d, dev)
        if w.logits_given:
            r["logits"] = dinp["logits"][:d.T].contiguous()
        out = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
        if noalloc:
            lm.forward_noalloc(d, x, dinp, w.logits_given, r, out)
        else:
            ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
            lm.forward(d, x, dinp, w.logits_given, r, out, ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}))
    return res


def _same(a, b, what):
    assert np.array_equal(a[0], b[0]), f"{what}: outputs differ"
    for k in a[1]:
        assert np.array_equal(a[1][k], b[1][k]), f"{what}: {k} differs"
    log(f"{what}: no-alloc call equals lmoe_forward")


@pytest.mark.parametrize("name,Ts", [
    ("ragged", (37, 9, 1)),          # grouped, grouped, single-token kernel
    ("ragged_skew", (509, 100)),     # given logits
])
def test_noalloc_matches_forward_on_shrinking_inputs(lm, dev, name, Ts):
    w0 = get_workload(name)
    inp = gen_all(w0)
    dinp = upload(inp, dev)
    xs = upload({"x": gen_x(w0)}, dev)["x"]
    for T in Ts:
        w = w0.with_T(T)
        a, b = _both(lm, dev, w, dinp, xs[:T].contiguous())
        _same(a, b, f"{name} T={T}")


def test_noalloc_k3_decode_after_batch(lm, dev):
    """Kimi-K3 widths: 24 tokens (grouped path), then one token (the
    single-token kernel, whose counters sit in the shared scratch)."""
    w0 = get_workload("decode")
    inp = gen_all(w0)
    dinp = upload(inp, dev)
    xs = upload({"x": gen_x(w0.with_T(24))}, dev)["x"]
    for T in (24, 1):
        w = w0.with_T(T)
        a, b = _both(lm, dev, w, dinp, xs[:T].contiguous())
        _same(a, b, f"K3 T={T}")

"""Pins of the oracle's MoE block (input step and tail around the layer:
TokenSpeed sections 4.2-4.4 and 6) against facts that do not come from the
oracle itself: a torch float64 statement that multiplies by the three input
projections as separate matrices (with W_in assembled here, row by row, from
the layout reading), torch's own rms_norm, closed forms of the tail, and
special cases of the whole block. A slip such as swapped gate and up rows, a
wrong group offset, a missing epsilon or residual, or the shared output not
rounded to bf16 fails at least one of them."""
import numpy as np
import pytest

import oracle as O


def _bits(rng, shape, std=1.0, mean=0.0):
    return O.bf16_from_f64(rng.normal(mean, std, size=shape))


def _assemble_w_in(wr, wl, gates, ups):
    """W_in row by row from separate matrices: router rows, latent rows, then
    per shared expert 16 gate rows followed by the 16 up rows of the same
    columns."""
    rows = list(wr) + list(wl)
    for g, u in zip(gates, ups):
        for j in range(g.shape[0] // 16):
            rows += list(g[16 * j:16 * j + 16])
            rows += list(u[16 * j:16 * j + 16])
    return np.array(rows, dtype=np.uint16)


def test_shared_gate_up_rows_hand_listed():
    gate, up = O.shared_gate_up_rows(E=4, L=8, S=2, Is=32)
    b = 12
    assert gate[0].tolist() == list(range(b, b + 16)) + list(range(b + 32, b + 48))
    assert up[0].tolist() == list(range(b + 16, b + 32)) + list(range(b + 48, b + 64))
    assert gate[1].tolist() == [r + 64 for r in gate[0].tolist()]
    # every row after the router and latent rows is used exactly once
    used = np.sort(np.concatenate([gate.ravel(), up.ravel()]))
    assert used.tolist() == list(range(b, b + 128))


@pytest.mark.parametrize("S", [0, 1, 2])
def test_moe_input_matches_separate_projections(S):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(30 + S)
    T, H, E, L, Is = 7, 96, 8, 32, 48
    u = _bits(rng, (T, H))
    wr = _bits(rng, (E, H), 0.1)
    wl = _bits(rng, (L, H), 0.1)
    gates = [_bits(rng, (Is, H), 0.1) for _ in range(S)]
    ups = [_bits(rng, (Is, H), 0.1) for _ in range(S)]
    res = O.moe_input(u, _assemble_w_in(wr, wl, gates, ups), E, L, S, Is)

    def t(b):
        return torch.from_numpy(O.f64_from_bf16(b))

    ut = t(u)
    assert np.array_equal(res["logits"], (ut @ t(wr).T).to(torch.float32).numpy())
    assert np.array_equal(res["x"], O.bf16_from_f64((ut @ t(wl).T).numpy()))
    assert res["h"].shape == (T, S * Is)
    for s in range(S):
        h = torch.nn.functional.silu(ut @ t(gates[s]).T) * (ut @ t(ups[s]).T)
        assert np.array_equal(res["h"][:, s * Is:(s + 1) * Is], O.bf16_from_f64(h.numpy()))


def test_rms_norm_matches_torch_and_closed_forms():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(40)
    L = 160
    r = _bits(rng, (9, L), 3.0)
    r[1] = O.bf16_from_f64(np.full(L, 0.75))           # constant row
    r[2] = 0                                            # zero row
    r[3] = O.bf16_from_f64(rng.normal(0, 1e-4, L))      # rms near sqrt(eps)
    gamma = _bits(rng, (L,), 0.1, 1.0)
    got = O.rms_norm(r, gamma)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(O.f64_from_bf16(r)), (L,),
                                       weight=torch.from_numpy(O.f64_from_bf16(gamma)),
                                       eps=1e-6)
    assert np.array_equal(got, O.bf16_from_f64(ref.numpy()))
    g = O.f64_from_bf16(gamma)
    assert np.array_equal(got[1], O.bf16_from_f64(0.75 / np.sqrt(0.75 ** 2 + 1e-6) * g))
    assert not O.f64_from_bf16(got[2]).any()
    assert O.RMS_EPS == 1e-6


def test_moe_tail_matches_torch_and_closed_forms():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(50)
    T, L, H, SIs = 6, 64, 96, 64
    routed = _bits(rng, (T, L))
    h = _bits(rng, (T, SIs))
    gamma = _bits(rng, (L,), 0.1, 1.0)
    w_up = _bits(rng, (H, L), 0.1)
    w_sd = _bits(rng, (H, SIs), 0.1)
    resid = _bits(rng, (T, H))
    got = O.moe_tail(routed, h, gamma, w_up, w_sd, resid)

    def t(b):
        return torch.from_numpy(O.f64_from_bf16(b))

    n = torch.nn.functional.rms_norm(t(routed), (L,), weight=t(gamma), eps=1e-6)
    n = t(O.bf16_from_f64(n.numpy()))
    sh = t(O.bf16_from_f64((t(h) @ t(w_sd).T).numpy()))
    out = n @ t(w_up).T + sh + t(resid)
    assert np.allclose(got["out64"], out.numpy(), rtol=1e-12, atol=1e-12)
    assert np.array_equal(got["out"], O.bf16_from_f64(out.numpy()))
    assert np.array_equal(got["sh"], O.bf16_from_f64((t(h) @ t(w_sd).T).numpy()))
    # a zero routed result leaves the shared output plus the residual
    z = O.moe_tail(np.zeros_like(routed), h, gamma, w_up, w_sd, resid)
    assert np.array_equal(z["out"], O.bf16_from_f64(
        O.f64_from_bf16(got["sh"]) + O.f64_from_bf16(resid)))
    # zero shared activations: the shared partial is exactly zero
    z = O.moe_tail(routed, np.zeros_like(h), gamma, w_up, w_sd, resid)
    assert not O.f64_from_bf16(z["sh"]).any()
    # with a zero residual and a zero routed result, out is exactly the
    # shared partial (its bf16 rounding before the sum is checked by the
    # torch statement above)
    z = O.moe_tail(np.zeros_like(routed), h, gamma, w_up, w_sd, np.zeros_like(resid))
    assert np.array_equal(z["out"], z["sh"])


def _block_inputs(seed, T=5, H=64, L=64, E=8, k=2, I=64, S=1, Is=32):
    rng = np.random.default_rng(seed)
    ex = {
        "gate_q": rng.integers(0, 256, size=(E, I, L // 2)).astype(np.uint8),
        "up_q": rng.integers(0, 256, size=(E, I, L // 2)).astype(np.uint8),
        "down_q": rng.integers(0, 256, size=(E, L, I // 2)).astype(np.uint8),
        "gate_s": rng.integers(122, 128, size=(E, I, L // 32)).astype(np.uint8),
        "up_s": rng.integers(122, 128, size=(E, I, L // 32)).astype(np.uint8),
        "down_s": rng.integers(122, 128, size=(E, L, I // 32)).astype(np.uint8),
    }
    return dict(u=_bits(rng, (T, H)), residual=_bits(rng, (T, H)),
                w_in=_bits(rng, (E + L + 2 * S * Is, H), 0.1), experts=ex,
                gamma=_bits(rng, (L,), 0.1, 1.0), w_up=_bits(rng, (H, L), 0.1),
                w_sd=_bits(rng, (H, S * Is), 0.1), E=E, L=L, S=S, Is=Is, k=k)


def _run_block(b, **kw):
    return O.block_forward(b["u"], b["residual"], b["w_in"], b["experts"], b["gamma"],
                           b["w_up"], b["w_sd"], b["E"], b["L"], b["S"], b["Is"], b["k"], **kw)


def test_block_with_silent_experts_is_shared_plus_residual():
    """Zero gate codes: every routed h is zero, so the routed result, its
    normalised form and its up-projection vanish, and the block's output is
    bf16(sh + residual) whatever the routing."""
    b = _block_inputs(60)
    b["experts"]["gate_q"][:] = 0
    res = _run_block(b)
    assert not O.f64_from_bf16(res["routed"]["out"]).any()
    sh = O.f64_from_bf16(res["tail"]["sh"])
    assert np.array_equal(res["out"], O.bf16_from_f64(sh + O.f64_from_bf16(b["residual"])))


def test_block_routes_on_the_input_steps_logits():
    """The routing inside the block is the top-k of the input step's router
    scores, the routed layer reads the input step's latent rows, and given
    logits replace the scores for routing only."""
    b = _block_inputs(61, T=6, E=16, k=3)
    res = _run_block(b)
    lg = res["input"]["logits"]
    assert np.array_equal(res["routed"]["idx"], O.topk_select(lg, b["k"]))
    # different logits: a reversed expert order changes the selection
    flipped = np.ascontiguousarray(lg[:, ::-1])
    res2 = _run_block(b, logits=flipped)
    assert np.array_equal(res2["routed"]["idx"], O.topk_select(flipped, b["k"]))
    assert np.array_equal(res2["input"]["x"], res["input"]["x"])
    assert not np.array_equal(res2["routed"]["idx"], res["routed"]["idx"])

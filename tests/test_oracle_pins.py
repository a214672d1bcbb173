"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against one of: the format definition of E2M1 /
E8M0 / E4M3 written out with exact rationals, hand-worked fixtures under
tests/golden/, brute force on tiny inputs, independent library routines
(numpy sorting and counting, scipy's softmax, torch's float32->bfloat16 and
float32->float8_e4m3fn conversions), closed-form special cases of the GLU FFN, and invariants of the
layer (expert relabelling, identical experts, token permutation, scaling of
the down projection). Each is chosen so that a plausible slip in the oracle
(a swapped nibble, a dropped shared expert, a transposed weight, a reversed
tie rule, a missing bf16 rounding) fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import get_workload, gen_all, gen_logits, gen_expert

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def _e2m1_from_bits(c: int) -> Fraction:
    """E2M1 by its bit fields: s | e1 e0 | m, exponent bias 1, e=0 subnormal."""
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    if e == 0:
        mag = Fraction(m, 2)
    else:
        mag = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def test_e2m1_table_matches_bit_field_definition():
    t = O.e2m1_table()
    for c in range(16):
        assert Fraction(float(t[c])) == _e2m1_from_bits(c), c
    # code 8 is negative zero
    assert t[8] == 0.0 and math.copysign(1.0, t[8]) < 0


def test_e2m1_table_matches_golden_grid():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_grid.txt"))
            if l.strip() and not l.startswith("#")]
    t = O.e2m1_table()
    assert len(rows) == 16
    for code, val in rows:
        v = float(val)
        assert t[int(code)] == v
        assert math.copysign(1.0, t[int(code)]) == math.copysign(1.0, v)


def test_e8m0_scale_closed_form():
    b = np.arange(256)
    s = O.e8m0_scale(b)
    for i in range(255):
        assert Fraction(float(s[i])) == Fraction(2) ** (i - 127)
    assert np.isnan(s[255])


def test_dequant_exhaustive_codes_and_scales():
    """All 16 codes x 256 exponents, in one 32-wide block per exponent."""
    # Row b holds one block of 32 elements with scale byte b; element j has code j % 16.
    N, K = 256, 32
    codes = np.tile(np.arange(32) % 16, (N, 1)).astype(np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = np.arange(256, dtype=np.uint8).reshape(N, 1)
    v = O.dequant_mxfp4(q, s, N, K)
    for b in range(256):
        for j in range(32):
            got = v[b, j]
            if b == 255:
                assert np.isnan(got)
                continue
            want = _e2m1_from_bits(j % 16) * Fraction(2) ** (b - 127)
            assert Fraction(float(got)) == want, (b, j)


def test_dequant_nibble_order_and_scale_direction():
    """Element 2m is the low nibble of byte m; scales run along the row (K)."""
    N, K = 3, 64
    q = np.zeros((N, K // 2), np.uint8)
    q[1, 5] = 0x72         # elements 10 (low nibble = 2 -> 1.0) and 11 (high = 7 -> 6.0)
    s = np.full((N, K // 32), 127, np.uint8)
    s[1, 0] = 128          # first block of row 1 doubled
    s[2, 1] = 125          # second block of row 2 only
    q[2, 20] = 0x09        # element 40 (low nibble 9 -> -0.5), in the second block
    v = O.dequant_mxfp4(q, s, N, K)
    assert v[1, 10] == 2.0 and v[1, 11] == 12.0
    assert v[2, 40] == -0.5 * 0.25
    nz = np.argwhere(v != 0)
    assert sorted(map(tuple, nz)) == [(1, 10), (1, 11), (2, 40)]


def _bf16_exact_bits(val: Fraction) -> int:
    """bf16 encoding of a value with at most 8 significant bits (no rounding)."""
    if val == 0:
        return 0
    sign = 0x8000 if val < 0 else 0
    a = abs(val)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if e > 127:
        return sign | 0x7F80
    if e < -126:
        q = a / Fraction(2) ** -133
        assert q.denominator == 1
        return sign | int(q)
    frac = a / Fraction(2) ** e - 1
    f = frac * 128
    assert f.denominator == 1
    return sign | ((e + 127) << 7) | int(f)


def test_bf16_rounding_of_every_dequantised_value():
    for b in range(255):
        for c in range(16):
            val = _e2m1_from_bits(c) * Fraction(2) ** (b - 127)
            fv = -0.0 if c == 8 else float(val)
            got = int(O.bf16_from_f64(np.array([fv]))[0])
            want = 0x8000 if c == 8 else _bf16_exact_bits(val)
            assert got == want, (c, b, hex(got), hex(want))


def test_dequant_golden_cases():
    path = os.path.join(GOLDEN, "mxfp4_bf16_cases.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        c, b, h = line.split()
        q = np.zeros((1, 16), np.uint8)
        q[0, 0] = int(c)
        s = np.array([[int(b)]], np.uint8)
        v = O.dequant_mxfp4(q, s, 1, 32)[0, 0]
        bits = int(O.bf16_from_f64(np.array([v]))[0])
        if h == "nan":
            assert np.isnan(v)
        else:
            assert bits == int(h, 16), (c, b, hex(bits), h)
        n += 1
    assert n >= 15


def test_bf16_rounding_matches_torch_on_float32_inputs():
    """torch's float32 -> bfloat16 conversion is round-to-nearest-even; on float32
    inputs the oracle's float64 rounding must agree bit for bit (ties, subnormals,
    overflow, signed zeros included)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties at the bf16 rounding point
    bits[:50000] = (bits[:50000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    bits[50000:60000] = (bits[50000:60000] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    extra = np.array([0.0, -0.0, 3.3895313892515355e38, 3.39e38, -3.4e38, 1e-40, -1e-45,
                      1.1754942e-38, 9.2e-41], np.float32)
    f32 = np.concatenate([f32, extra])
    ours = O.bf16_from_f64(f32.astype(np.float64))
    theirs = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mismatch = np.nonzero(ours != theirs)[0]
    assert mismatch.size == 0, [(float(f32[i]), hex(ours[i]), hex(theirs[i])) for i in mismatch[:5]]


def test_bf16_special_values():
    v = np.array([np.inf, -np.inf, np.nan, 1e300, -1e300, 0.0, -0.0, 2.0 ** -140])
    b = O.bf16_from_f64(v)
    assert list(b[:2]) == [0x7F80, 0xFF80]
    assert (b[2] & 0x7F80) == 0x7F80 and (b[2] & 0x7F) != 0
    assert list(b[3:7]) == [0x7F80, 0xFF80, 0x0000, 0x8000]
    assert b[7] == 0   # below half the smallest subnormal


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def _precedes(la, a, lb, b) -> bool:
    """a before b: larger logit first; NaN after every number; ties by index."""
    na, nb = math.isnan(la), math.isnan(lb)
    if na != nb:
        return nb
    if na and nb:
        return a < b
    if la != lb:
        return la > lb
    return a < b


def _brute_topk(row, k):
    remaining = list(range(len(row)))
    out = []
    for _ in range(k):
        best = remaining[0]
        for e in remaining[1:]:
            if _precedes(float(row[e]), e, float(row[best]), best):
                best = e
        out.append(best)
        remaining.remove(best)
    return out


@pytest.mark.parametrize("E,k", [(8, 1), (8, 3), (8, 8), (32, 4), (40, 16), (17, 5)])
def test_topk_brute_force_with_heavy_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    pool = np.array([1.5, 1.5, 0.0, -0.0, -2.0, 3.0, np.nan, -np.inf, np.inf, 0.25], np.float32)
    lg = rng.choice(pool, size=(60, E)).astype(np.float32)
    lg[:20] = rng.normal(size=(20, E)).astype(np.float32)
    idx = O.topk_select(lg, k)
    for t in range(lg.shape[0]):
        assert list(idx[t]) == _brute_topk(lg[t], k), t


def test_topk_k1_is_first_argmax_and_kE_is_stable_sort():
    rng = np.random.default_rng(7)
    lg = rng.integers(-3, 4, size=(50, 23)).astype(np.float32)
    assert np.array_equal(O.topk_select(lg, 1)[:, 0], np.argmax(lg, axis=1))
    full = O.topk_select(lg, 23)
    assert np.array_equal(full, np.argsort(-lg, axis=1, kind="stable"))


def test_topk_skewed_tie_groups_take_lowest_ids():
    """In the skewed workload a tied group of 32 experts sits above every other
    logit of its token, so the top 16 are the group's 16 lowest expert ids, in
    ascending order (the lower-index tie rule)."""
    w = get_workload("ragged_skew")
    lg = gen_logits(w)
    k = w.dims.k
    idx = O.topk_select(lg, k)
    n_tied = 0
    for t in range(lg.shape[0]):
        top = lg[t].max()
        grp = np.nonzero(lg[t] == top)[0]
        if grp.size > k:
            n_tied += 1
            assert list(idx[t]) == sorted(grp)[:k]
    assert n_tied == int(round(w.tie_frac * w.dims.T))


def test_softmax_weights_against_scipy_and_closed_forms():
    scipy_special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(3)
    lg = rng.normal(size=(40, 30)).astype(np.float32)
    idx = O.topk_select(lg, 6)
    w = O.softmax_selected(lg, idx)
    sel = np.take_along_axis(lg.astype(np.float64), idx.astype(np.int64), axis=1)
    ref = scipy_special.softmax(sel, axis=1)
    assert np.array_equal(w, ref.astype(np.float32)) or np.max(np.abs(w - ref)) < 2e-7
    # weights follow the order of the logits
    assert np.all(np.diff(w, axis=1) <= 0)
    # k = 1 gives exactly 1; equal logits give exactly fp32(1/k)
    assert np.all(O.softmax_selected(lg, O.topk_select(lg, 1)) == 1.0)
    eq = np.zeros((3, 16), np.float32)
    for k in (2, 4, 5, 16):
        wk = O.softmax_selected(eq, O.topk_select(eq, k))
        assert np.all(wk == np.float32(1.0 / k))


def test_router_logits_one_hot_and_ones():
    L, E = 64, 12
    rng = np.random.default_rng(1)
    wr = O.bf16_from_f64(rng.normal(0, 0.02, size=(E, L)))
    x = np.zeros((L, L), np.uint16)
    for t in range(L):
        x[t, t] = 0x3F80          # 1.0
    lg = O.router_logits(x, wr)
    # token t picks column t of W: the logit of expert e is W[e, t]
    assert np.array_equal(lg, O.f64_from_bf16(wr).T.astype(np.float32))
    # x = 1 and W = 0.5 everywhere: logits are exactly L/2
    ones = np.full((2, L), 0x3F80, np.uint16)
    half = np.full((E, L), 0x3F00, np.uint16)
    assert np.all(O.router_logits(ones, half) == L / 2)


def test_permutation_against_numpy_stable_argsort():
    rng = np.random.default_rng(11)
    for T, k, E in [(1, 16, 896), (37, 6, 48), (200, 8, 10), (5, 5, 5)]:
        lg = rng.normal(size=(T, E)).astype(np.float32)
        lg[:, : min(3, E)] += 2.0        # crowd a few experts
        idx = O.topk_select(lg, k)
        counts, offsets, perm, inv = O.permute_routes(idx, E)
        flat = idx.ravel()
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert np.array_equal(offsets[1:], np.cumsum(np.bincount(flat, minlength=E)))
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(inv[perm], np.arange(T * k))


# ----------------------------------------------------------------------------
# Experts and the whole layer
# ----------------------------------------------------------------------------

def _pack(codes: np.ndarray) -> np.ndarray:
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_glu_one_hot_input_reads_a_weight_column():
    """Scale 127 and x = e_l: g and u are column l of the dequantised weights."""
    L, I = 64, 32
    rng = np.random.default_rng(2)
    gq = _pack(rng.integers(0, 16, size=(I, L)).astype(np.uint8))
    uq = _pack(rng.integers(0, 16, size=(I, L)).astype(np.uint8))
    s = np.full((I, L // 32), 127, np.uint8)
    gate = O.dequant_mxfp4(gq, s, I, L)
    up = O.dequant_mxfp4(uq, s, I, L)
    down = np.eye(L, I)
    for l in (0, 17, 63):
        x = np.zeros((1, L))
        x[0, l] = 1.0
        h_bits, y = O.glu_ffn(x, gate, up, down)
        g = gate[:, l]
        u = up[:, l]
        want = g / (1 + np.exp(-g)) * u
        # compare values: a sum of +0 products is +0 where the element-wise
        # product of a -0 code is -0
        assert np.array_equal(O.f64_from_bf16(h_bits[0]), O.f64_from_bf16(O.bf16_from_f64(want)))
        # down = identity on the first I coordinates
        assert np.array_equal(y[0, :I], O.f64_from_bf16(h_bits[0]))
        assert np.all(y[0, I:] == 0)


def test_glu_closed_form_all_ones():
    """All codes 2 (1.0) with scale 127, x = 1: g = u = L exactly, so
    h = bf16(L^2 / (1 + e^-L)) = L^2 for L = 64, and with down all 1.0,
    every output is I * L^2."""
    L, I = 64, 96
    gate = np.ones((I, L))
    q = _pack(np.full((I, L), 2, np.uint8))
    s = np.full((I, L // 32), 127, np.uint8)
    assert np.array_equal(O.dequant_mxfp4(q, s, I, L), gate)
    qd = _pack(np.full((L, I), 1, np.uint8))       # 0.5 ...
    sd = np.full((L, I // 32), 128, np.uint8)      # ... times 2
    down = O.dequant_mxfp4(qd, sd, L, I)
    assert np.all(down == 1.0)
    h_bits, y = O.glu_ffn(np.ones((2, L)), gate, gate, down)
    assert np.all(O.f64_from_bf16(h_bits) == L * L)
    assert np.all(y == I * L * L)


def _small_layer(seed=0, T=9, L=64, E=6, k=3, I=64, S=2, Is=32):
    rng = np.random.default_rng(seed)
    x = O.bf16_from_f64(rng.normal(size=(T, L)))
    wr = O.bf16_from_f64(rng.normal(0, 0.1, size=(E, L)))
    ex = {
        "gate_q": rng.integers(0, 256, size=(E, I, L // 2)).astype(np.uint8),
        "up_q": rng.integers(0, 256, size=(E, I, L // 2)).astype(np.uint8),
        "down_q": rng.integers(0, 256, size=(E, L, I // 2)).astype(np.uint8),
        "gate_s": rng.integers(122, 128, size=(E, I, L // 32)).astype(np.uint8),
        "up_s": rng.integers(122, 128, size=(E, I, L // 32)).astype(np.uint8),
        "down_s": rng.integers(122, 128, size=(E, L, I // 32)).astype(np.uint8),
    }
    sh = {
        "sh_gate": O.bf16_from_f64(rng.normal(0, 0.1, size=(S, Is, L))),
        "sh_up": O.bf16_from_f64(rng.normal(0, 0.1, size=(S, Is, L))),
        "sh_down": O.bf16_from_f64(rng.normal(0, 0.1, size=(S, L, Is))),
    }
    return x, wr, ex, sh


def _ref_dequant(q, s, N, K):
    """Element-wise dequantisation from the bit-field definition (slow)."""
    out = np.empty((N, K))
    for n in range(N):
        for kk in range(K):
            byte = int(q[n, kk // 2])
            code = (byte >> 4) if kk % 2 else (byte & 15)
            out[n, kk] = float(_e2m1_from_bits(code) * Fraction(2) ** (int(s[n, kk // 32]) - 127))
    return out


def test_forward_matches_independent_torch_layer():
    """A second, independent statement of the layer in torch float64 (element-wise
    dequantisation from bit fields, brute-force top-k, scipy softmax, torch SiLU,
    per-route loop, shared experts) must agree with the oracle."""
    torch = pytest.importorskip("torch")
    scipy_special = pytest.importorskip("scipy.special")
    x, wr, ex, sh = _small_layer()
    T, L = x.shape
    E, I = ex["gate_q"].shape[:2]
    k = 3
    res = O.forward(x, wr, ex, sh, k)

    xt = torch.from_numpy(O.f64_from_bf16(x))
    lg = (xt @ torch.from_numpy(O.f64_from_bf16(wr)).T).to(torch.float32).numpy()
    assert np.array_equal(lg, res["logits"])
    W = {}
    for e in range(E):
        W[e] = (torch.from_numpy(_ref_dequant(ex["gate_q"][e], ex["gate_s"][e], I, L)),
                torch.from_numpy(_ref_dequant(ex["up_q"][e], ex["up_s"][e], I, L)),
                torch.from_numpy(_ref_dequant(ex["down_q"][e], ex["down_s"][e], L, I)))

    def bf16_round(t):
        return torch.from_numpy(O.f64_from_bf16(O.bf16_from_f64(t.numpy())))

    out = torch.zeros(T, L, dtype=torch.float64)
    for t in range(T):
        sel = _brute_topk(lg[t], k)
        assert list(res["idx"][t]) == sel
        wts = scipy_special.softmax(lg[t, sel].astype(np.float64)).astype(np.float32)
        for j, e in enumerate(sel):
            G, U, D = W[e]
            h = bf16_round(torch.nn.functional.silu(G @ xt[t]) * (U @ xt[t]))
            out[t] += float(wts[j]) * (D @ h)
        for s in range(sh["sh_gate"].shape[0]):
            G = torch.from_numpy(O.f64_from_bf16(sh["sh_gate"][s]))
            U = torch.from_numpy(O.f64_from_bf16(sh["sh_up"][s]))
            D = torch.from_numpy(O.f64_from_bf16(sh["sh_down"][s]))
            h = bf16_round(torch.nn.functional.silu(G @ xt[t]) * (U @ xt[t]))
            out[t] += D @ h
    ref = out.numpy()
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(res["out64"] - ref)) <= 1e-9 * scale
    assert np.array_equal(res["out"], O.bf16_from_f64(res["out64"]))


def test_zero_gate_codes_leave_only_shared_experts():
    x, wr, ex, sh = _small_layer(seed=4)
    ex["gate_q"][:] = 0
    full = O.forward(x, wr, ex, sh, 3)
    only_sh = O.forward(x, wr, ex, {k: v[:0] for k, v in sh.items()}, 3)
    assert np.all(only_sh["out64"] == 0)
    sh0 = {k: v[:1] for k, v in sh.items()}
    sh1 = {k: v[1:] for k, v in sh.items()}
    a = O.forward(x, wr, ex, sh0, 3)["out64"]
    b = O.forward(x, wr, ex, sh1, 3)["out64"]
    assert np.allclose(full["out64"], a + b, rtol=0, atol=1e-12 * np.abs(full["out64"]).max())
    assert np.abs(a).max() > 0 and np.abs(b).max() > 0


def test_identical_experts_reduce_to_one_expert():
    """With every routed expert identical, the routed part equals that single
    expert's output whatever the routing (the weights sum to 1)."""
    x, wr, ex, sh = _small_layer(seed=6)
    for key in ex:
        ex[key][:] = ex[key][0]
    res = O.forward(x, wr, ex, {k: v[:0] for k, v in sh.items()}, 3)
    gate = O.dequant_mxfp4(ex["gate_q"][0], ex["gate_s"][0], 64, 64)
    up = O.dequant_mxfp4(ex["up_q"][0], ex["up_s"][0], 64, 64)
    down = O.dequant_mxfp4(ex["down_q"][0], ex["down_s"][0], 64, 64)
    _, y = O.glu_ffn(O.f64_from_bf16(x), gate, up, down)
    wsum = res["w"].astype(np.float64).sum(axis=1, keepdims=True)
    assert np.allclose(res["out64"], wsum * y, rtol=1e-12, atol=1e-9)
    assert np.allclose(wsum, 1.0, atol=1e-6)


def test_relabelling_experts_leaves_output_unchanged():
    x, wr, ex, sh = _small_layer(seed=8, E=7)
    base = O.forward(x, wr, ex, sh, 3)
    p = np.random.default_rng(0).permutation(7)       # new label of old expert e is inv[e]
    ex2 = {k: v[p] for k, v in ex.items()}
    wr2 = wr[p]                                       # router rows follow their experts
    res = O.forward(x, wr2, ex2, sh, 3)
    assert np.array_equal(res["out"], base["out"])
    assert np.array_equal(p[res["idx"]], base["idx"])


def test_token_permutation_and_down_scale():
    x, wr, ex, sh = _small_layer(seed=9)
    base = O.forward(x, wr, ex, {k: v[:0] for k, v in sh.items()}, 3)
    p = np.random.default_rng(1).permutation(x.shape[0])
    res = O.forward(x[p], wr, ex, {k: v[:0] for k, v in sh.items()}, 3)
    assert np.array_equal(res["out"], base["out"][p])
    ex2 = dict(ex)
    ex2["down_s"] = (ex["down_s"] + 1).astype(np.uint8)     # doubles every down weight
    res2 = O.forward(x, wr, ex2, {k: v[:0] for k, v in sh.items()}, 3)
    assert np.array_equal(res2["out64"], 2.0 * base["out64"])


def test_forward_tokens_subset_matches_full_forward():
    w = get_workload("tiny")
    d = gen_all(w)
    full = O.forward(d["x"], d["router_w"], d, d, w.dims.k)
    toks = [0, 5, 7]
    o64, ob = O.forward_tokens(d["x"], full["idx"], full["w"],
                               lambda e: gen_expert(w, e), d, w.dims.L, w.dims.I, toks)
    # BLAS may block a sub-batch differently: float64 sums agree to rounding
    ref = full["out64"][toks]
    assert np.max(np.abs(o64 - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.mean(ob == full["out"][toks]) > 0.999


# ----------------------------------------------------------------------------
# Quantised activations (E4M3 / E2M1 elements, one E8M0 scale per 32)
# ----------------------------------------------------------------------------

def _e4m3_from_bits(c: int):
    """E4M3 by its bit fields, exact; None for the NaN codes."""
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return None
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def test_e4m3_table_matches_bit_fields_and_torch():
    import torch
    t = O.e4m3_table()
    for c in range(256):
        ref = _e4m3_from_bits(c)
        if ref is None:
            assert np.isnan(t[c])
        else:
            assert t[c] == float(ref) and math.copysign(1, t[c]) == (-1 if c & 0x80 else 1)
    via_torch = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    tt = via_torch.to(torch.float64).numpy()
    assert np.array_equal(np.isnan(tt), np.isnan(t))
    assert np.array_equal(tt[~np.isnan(tt)], t[~np.isnan(t)])
    assert t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9


def _brute_round(q: float, fmt: str) -> int:
    """Nearest grid magnitude by exhaustive comparison, ties to the even
    code, saturating; the sign bit from q's sign."""
    mags = [_e2m1_from_bits(c) for c in range(8)] if fmt == "e2m1" else \
        [_e4m3_from_bits(c) for c in range(127)]
    a = abs(Fraction(q))
    if a >= mags[-1]:
        code = len(mags) - 1
    else:
        best = min(abs(m - a) for m in mags)
        near = [i for i, m in enumerate(mags) if abs(m - a) == best]
        code = near[0] if len(near) == 1 else [i for i in near if i % 2 == 0][0]
    sign = (0x8 if fmt == "e2m1" else 0x80) if math.copysign(1, q) < 0 else 0
    return code | sign


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_round_to_format_brute_force(fmt):
    rng = np.random.default_rng(5)
    mags = np.array([float(_e2m1_from_bits(c)) for c in range(8)]) if fmt == "e2m1" else \
        O.e4m3_table()[:127]
    mids = (mags[:-1] + mags[1:]) / 2
    top = mags[-1]
    q = np.concatenate([mids, -mids, mags, -mags, [0.0, -0.0, top * 1.01, -top * 3, top * 100],
                        rng.normal(size=200) * top / 3, rng.uniform(-top, top, size=200),
                        np.ldexp(rng.uniform(1, 2, size=60), rng.integers(-12, 2, size=60))])
    got = O.round_to_format(q, fmt)
    want = np.array([_brute_round(float(v), fmt) for v in q], np.uint8)
    assert np.array_equal(got, want)


def test_round_to_format_e4m3_matches_torch_cast():
    import torch
    rng = np.random.default_rng(6)
    q = np.concatenate([rng.uniform(-448, 448, size=4000), rng.normal(size=4000) * 0.01,
                        (O.e4m3_table()[:126] + O.e4m3_table()[1:127]) / 2])
    q32 = q.astype(np.float32)
    ref = torch.from_numpy(q32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.round_to_format(q32.astype(np.float64), "e4m3"), ref)


def test_mx_quantize_golden_cases():
    with open(os.path.join(GOLDEN, "mx_act_cases.txt")) as f:
        lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) == 8
    for fmt, byte, *pairs in lines:
        vals = [float(p.split(":")[0]) for p in pairs]
        codes = [int(p.split(":")[1]) for p in pairs]
        block = np.zeros((1, 32))
        block[0, :len(vals)] = vals
        c, e = O.mx_quantize(block, fmt)
        assert int(e[0, 0]) == int(byte), (fmt, byte, e)
        assert c[0, :len(codes)].tolist() == codes, (fmt, pairs, c[0, :len(codes)])
        assert not c[0, len(codes):].any()


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_mx_quantize_properties(fmt):
    """Scale exponent by exhaustive search (the largest element lands in the
    top binade of the element grid), error within half a grid step of the
    scaled value, and quantising the dequantised values reproduces them."""
    rng = np.random.default_rng(7)
    v = rng.normal(size=(40, 64)) * np.ldexp(1.0, rng.integers(-20, 20, size=(40, 1)))
    v[3] = 0.0
    v = O.f64_from_bf16(O.bf16_from_f64(v))
    codes, exps = O.mx_quantize(v, fmt)
    emax = O.ACT_EMAX[fmt]
    top = 6.0 if fmt == "e2m1" else 448.0
    for r in range(v.shape[0]):
        for b in range(2):
            blk = v[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            X = int(exps[r, b]) - 127
            if amax == 0:
                assert X == 0
                continue
            # the one X with 2^emax <= amax / 2^X < 2^(emax+1)
            cands = [x for x in range(-160, 160) if 2.0 ** emax <= amax / 2.0 ** x < 2.0 ** (emax + 1)]
            assert cands == [X]
    deq = O.mx_dequant(codes, exps, fmt)
    c2, e2 = O.mx_quantize(deq, fmt)
    assert np.array_equal(c2, codes) and np.array_equal(e2, exps)
    scale = np.repeat(O.e8m0_scale(exps), 32, axis=1)
    q = v / scale
    mags = np.sort(np.abs(O.format_values(np.arange(16 if fmt == "e2m1" else 127), fmt)))
    mags = np.unique(mags)
    # half the local grid step around each value (saturated values excepted)
    idx = np.clip(np.searchsorted(mags, np.abs(q)), 1, mags.size - 1)
    step = mags[idx] - mags[idx - 1]
    inside = np.abs(q) <= top
    assert np.all(np.abs(deq / scale - q)[inside] <= step[inside] / 2 + 1e-300)


def test_forward_e4m3_matches_torch_float8_layer():
    """The layer with E4M3 activations against an independent float64 torch
    statement that quantises through torch's float8_e4m3fn cast (per-block
    scale 2^(floor(log2 amax) - 8), values clamped to +-448 before the
    cast)."""
    import torch
    w = get_workload("tiny")
    d = w.dims
    inp = gen_all(w)
    ref = O.forward(inp["x"], inp["router_w"], inp, inp, d.k, act="e4m3")

    def q8(v):  # [m][K] float64 torch
        blk = v.reshape(v.shape[0], -1, 32)
        amax = blk.abs().amax(dim=2, keepdim=True)
        X = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 8,
                        torch.zeros_like(amax))
        sc = torch.pow(2.0, X)
        e = (blk / sc).clamp(-448, 448).to(torch.float32).to(torch.float8_e4m3fn)
        return (e.to(torch.float64) * sc).reshape(v.shape)

    x = torch.from_numpy(O.f64_from_bf16(inp["x"]))
    out = torch.zeros(d.T, d.L, dtype=torch.float64)
    idx, wts = ref["idx"], ref["w"].astype(np.float64)
    for t in range(d.T):
        for j in range(d.k):
            e = int(idx[t, j])
            ex = gen_expert(w, e)
            G = torch.from_numpy(O.dequant_mxfp4(ex["gate_q"], ex["gate_s"], d.I, d.L))
            U = torch.from_numpy(O.dequant_mxfp4(ex["up_q"], ex["up_s"], d.I, d.L))
            D = torch.from_numpy(O.dequant_mxfp4(ex["down_q"], ex["down_s"], d.L, d.I))
            xa = q8(x[t:t + 1])
            g, u = xa @ G.T, xa @ U.T
            hh = (g * torch.sigmoid(g) * u).to(torch.bfloat16).to(torch.float64)
            out[t] += wts[t, j] * (q8(hh) @ D.T)[0]
        for sidx in range(d.S):
            G = torch.from_numpy(O.f64_from_bf16(inp["sh_gate"][sidx]))
            U = torch.from_numpy(O.f64_from_bf16(inp["sh_up"][sidx]))
            D = torch.from_numpy(O.f64_from_bf16(inp["sh_down"][sidx]))
            g, u = x[t:t + 1] @ G.T, x[t:t + 1] @ U.T
            hh = (g * torch.sigmoid(g) * u).to(torch.bfloat16).to(torch.float64)
            out[t] += (hh @ D.T)[0]
    assert np.allclose(ref["out64"], out.numpy(), rtol=1e-12, atol=1e-12)
    # and the quantisation did something: the bf16 layer differs
    plain = O.forward(inp["x"], inp["router_w"], inp, inp, d.k)
    assert not np.allclose(plain["out64"], ref["out64"], rtol=1e-6, atol=0)


def test_forward_activation_formats_reduce_when_representable():
    """Tokens whose every 32-block is already an E2M1 block (grid values times
    a power of two, the block maximum in the top binade) give the same gate
    and up products in every activation format; zero-gate experts then leave
    the quantised layer equal to the plain one."""
    w = get_workload("tiny")
    d = w.dims
    inp = gen_all(w)
    rng = np.random.default_rng(9)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6.0])
    v = rng.choice(grid, size=(d.T, d.L)) * rng.choice([-1, 1], size=(d.T, d.L))
    v[:, ::32] = 6.0
    v = v * np.ldexp(1.0, rng.integers(-3, 3, size=(d.T, d.L // 32))).repeat(32, axis=1)
    x = O.bf16_from_f64(v)
    for fmt in ("e2m1", "e4m3"):
        assert np.array_equal(O.act_values(O.f64_from_bf16(x), fmt), O.f64_from_bf16(x))
    zero = dict(inp)
    zero["gate_q"] = np.zeros_like(inp["gate_q"])
    a = O.forward(x, inp["router_w"], zero, inp, d.k)
    for fmt in ("e2m1", "e4m3"):
        b = O.forward(x, inp["router_w"], zero, inp, d.k, act=fmt)
        assert np.array_equal(a["out"], b["out"])

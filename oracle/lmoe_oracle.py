"""Float64 CPU oracle of the LatentMoE MXFP4 (w4a16) routed-expert layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

What the layer computes, step by step, and where the pages state it:

  dequant   MXFP4 weights: E2M1 4-bit codes, one E8M0 power-of-two exponent
            per 32 consecutive values along the input dimension, bias 127
            (infervisor.ai "Bringing up Kimi-K3 on day zero", section "The
            model we hadn't run"; huggingface.co "Notes from an NVFP4 port of
            Kimi K3.1 Pro", introduction, which also states that the E2M1 grid
            is the one NVFP4 uses and that the exponent runs along columns).
  logits    router scores of each token over the 896 experts (dev48.org "Kimi
            K3 on AMD Instinct GPUs with TokenSpeed", section 4.3, router
            scores as one projection of the MoE input). Here the router reads
            the latent activations, as the workloads specify.
  top-k     16 of 896 experts per token (Bringing up Kimi-K3, "The model we
            hadn't run"; TokenSpeed section 4). Equal logits are broken toward
            the lower expert index, and the selected list is ordered by
            descending logit then ascending index. The block-oracle remark in
            Bringing up Kimi-K3, "Correctness before latency", is why only the
            selected set matters for the combine.
  weights   softmax over the selected logits (the workloads' gating rule; the
            pages do not state K3's router nonlinearity).
  permute   routes grouped by expert, stable in route order: counts, exclusive
            offsets, perm (position -> route), inverse (TokenSpeed section 4.1,
            sorting routes by expert so one weight panel serves several).
  experts   per route, a GLU FFN in the latent: g = x Gq^T, u = x Uq^T,
            h = bf16(silu(g) * u), y = h Dq^T (TokenSpeed section 4; the
            activation word printed on the pages is garbled, SiLU is used as the
            workloads state). Route partials stay in high precision (TokenSpeed
            section 4.3 sums route partials in FP32; here float64).
  shared    the same GLU with bf16 weights for each always-on shared expert,
            weight 1 (Bringing up Kimi-K3, "The model we hadn't run").
  combine   out[t] = bf16(sum_j w[t,j] y[t,j] + sum_s ysh[s,t]) in that order
            (TokenSpeed section 4.3, fused combine of the selected experts).
  block     around the layer, the MoE input step (router scores, latent
            input and shared gate/up from one packed projection of the hidden
            input, TokenSpeed section 4.3) and the tail (routed RMSNorm,
            latent -> hidden up-projection, plus the shared output and the
            residual, sections 4.2-4.3 and 6): moe_input, rms_norm, moe_tail,
            block_forward, with the readings stated at their definitions.

Readings where the pages are silent: element 2m of a row is the low nibble of
byte m; E8M0 byte 255 is NaN; NaN logits rank below -inf, equal NaNs by index;
-0 and +0 compare equal; h and out are rounded to bf16 nearest-even.

Every product x*w is exact in float64 (bf16 times a 2-significant-bit E2M1
value times a power of two), so the only deviation from exact arithmetic is
float64 summation and the stated bf16/fp32 roundings.

Quantised activations (optional, routed experts only). The pages list the
routed-expert GEMMs of their MI355X engine as FP8 activations with MXFP4
weights for small decode and MXFP4 activations with MXFP4 weights for prefill
(TokenSpeed, the precision table, row "Routed-expert GEMMs"); the shared
experts and the router stay bf16 (same table). The pages give no scale
granularity for the activations. Reading taken: the MX scheme the weights
already use, one E8M0 power-of-two scale per 32 consecutive values along K
for both element formats (FP8 E4M3 and FP4 E2M1). A block's scale exponent is
floor(log2(max |v|)) minus the element format's largest exponent (8 for E4M3,
2 for E2M1), clamped to the E8M0 range; a block of zeros takes 2^0. Each
element is v / 2^X rounded to the nearest representable value, ties to the
even code, saturating at the format's largest finite value (448, 6). The
gate/up input is the token's bf16 row; the down input is h after its bf16
rounding.
"""
from __future__ import annotations

from typing import Callable, Dict, Mapping, Optional, Sequence

import numpy as np

# Magnitudes of the E2M1 grid for codes 0..7; bit 3 of a code is the sign.
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E8M0_BIAS = 127


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def e2m1_table() -> np.ndarray:
    """Value of each of the 16 E2M1 codes (float64), code 8 is -0.0."""
    t = np.empty(16, np.float64)
    for c in range(16):
        mag = E2M1_MAGNITUDES[c & 7]
        t[c] = -mag if (c >> 3) & 1 else mag
    return t


def e8m0_scale(b) -> np.ndarray:
    """2**(b - 127) for E8M0 byte b; 255 encodes NaN."""
    b = np.asarray(b, dtype=np.int64)
    s = np.ldexp(np.ones(b.shape, np.float64), b - E8M0_BIAS)
    return np.where(b == 255, np.nan, s)


def dequant_mxfp4(q: np.ndarray, s: np.ndarray, N: int, K: int) -> np.ndarray:
    """Values of an [N][K] MXFP4 matrix, float64.

    q: uint8 [N][K/2], element k of row n in byte k//2, low nibble for even k.
    s: uint8 [N][K/32], exponent of elements 32j .. 32j+31 of row n.
    """
    q = np.asarray(q, np.uint8).reshape(N, K // 2)
    s = np.asarray(s, np.uint8).reshape(N, K // 32)
    codes = np.empty((N, K), np.uint8)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    vals = e2m1_table()[codes]
    scale = e8m0_scale(s)                          # [N][K/32]
    return vals * np.repeat(scale, 32, axis=1)


def f64_from_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_from_f64(v: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 (nearest, ties to even) and return the bit pattern.

    Full range: overflow to +-inf, bf16 subnormals, signed zeros, NaN.
    """
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    sign = np.where(np.signbit(v), 0x8000, 0).astype(np.uint16)
    a = np.abs(v)
    nan = np.isnan(v)
    inf = np.isinf(a)
    fin = ~(nan | inf)
    bits = np.zeros(v.shape, np.int64)
    with np.errstate(invalid="ignore", over="ignore"):
        # normal range: 8 significant bits
        m, e = np.frexp(np.where(fin, a, 1.0))        # a = m 2^e, m in [0.5, 1)
        q = np.rint(m * 256.0).astype(np.int64)       # 128..256, ties to even
        carry = q == 256
        q = np.where(carry, 128, q)
        e = np.where(carry, e + 1, e)
        biased = e + 126                              # bf16 exponent field
        normal_bits = (biased << 7) | (q - 128)
        # subnormal range: multiples of 2^-133
        sub_q = np.rint(np.ldexp(np.where(fin, a, 0.0), 133)).astype(np.int64)
        is_sub = a < 2.0 ** -126
        bits = np.where(is_sub, sub_q, normal_bits)
        bits = np.where(~is_sub & (biased >= 255), 0x7F80, bits)
    bits = np.where(inf, 0x7F80, bits)
    out[...] = (bits.astype(np.uint16) | sign)
    out[nan] = 0x7FC0
    return out


def f32_round(v: np.ndarray) -> np.ndarray:
    """float64 -> float32, nearest-even (IEEE conversion)."""
    return np.asarray(v, np.float64).astype(np.float32)


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, router_bits: np.ndarray) -> np.ndarray:
    """logits[t,e] = fp32(sum_l x[t,l] W[e,l]), float64 sum. W is [E][L]: one
    row of the router projection per expert."""
    x = f64_from_bf16(x_bits)
    wr = f64_from_bf16(router_bits)
    return f32_round(x @ wr.T)


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """First k experts of each row under the total order
    a before b  <=>  l_a > l_b  or  (l_a == l_b and a < b),
    compared as IEEE values (-0 == +0), NaN after every number.
    Returns int32 [T][k] listed in that order."""
    lg = np.asarray(logits, np.float32).astype(np.float64)
    T, E = lg.shape
    isnan = np.isnan(lg)
    val = np.where(isnan, 0.0, lg)
    val = np.where(val == 0.0, 0.0, val)     # -0 and +0 are the same key
    out = np.empty((T, k), np.int32)
    expert = np.arange(E)
    for t in range(T):
        order = np.lexsort((expert, -val[t], isnan[t]))
        out[t] = order[:k]
    return out


def softmax_selected(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected experts
    (l_0 the first, largest), in float64, stored as float32."""
    lg = np.asarray(logits, np.float32).astype(np.float64)
    sel = np.take_along_axis(lg, np.asarray(idx, np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return f32_round(z / z.sum(axis=1, keepdims=True))


def permute_routes(idx: np.ndarray, E: int):
    """Group routes r = t*k + j by expert, stable in r.

    Returns counts [E], offsets [E+1] (exclusive prefix sums), perm [T*k]
    (perm[pos] = r) and inv [T*k] (inv[r] = pos), all int32.
    Written as an explicit counting sort.
    """
    flat = np.asarray(idx, np.int64).ravel()
    R = flat.size
    counts = np.zeros(E, np.int64)
    for r in range(R):
        counts[flat[r]] += 1
    offsets = np.zeros(E + 1, np.int64)
    run = 0
    for e in range(E):
        offsets[e] = run
        run += counts[e]
    offsets[E] = run
    cursor = offsets[:E].copy()
    perm = np.empty(R, np.int64)
    inv = np.empty(R, np.int64)
    for r in range(R):
        e = flat[r]
        pos = cursor[e]
        cursor[e] += 1
        perm[pos] = r
        inv[r] = pos
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))


# ----------------------------------------------------------------------------
# Quantised activations (the reading in the module docstring)
# ----------------------------------------------------------------------------

ACT_FORMATS = ("bf16", "e4m3", "e2m1")
# largest exponent of a finite element value: E4M3 448 = 1.75 * 2^8, E2M1 6 = 1.5 * 2^2
ACT_EMAX = {"e4m3": 8, "e2m1": 2}


def e4m3_table() -> np.ndarray:
    """Value of each of the 256 FP8 E4M3 codes (float64): sign bit 7,
    exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 holds the
    subnormals m/8 * 2^-6; no infinities, and S.1111.111 is NaN."""
    t = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


def _magnitudes(fmt: str) -> np.ndarray:
    """Non-negative finite values of a format, indexed by magnitude code."""
    if fmt == "e2m1":
        return np.asarray(E2M1_MAGNITUDES, np.float64)
    return e4m3_table()[:127]          # codes 0..126: 0 .. 448


def round_to_format(q: np.ndarray, fmt: str) -> np.ndarray:
    """Codes of the values q (float64, finite) in an element format: the
    nearest representable magnitude, a tie to the even magnitude code,
    beyond the largest finite value that value; the sign bit from q's sign
    (so -0 and small negatives keep it). E2M1 codes are 4-bit (sign bit 3),
    E4M3 codes 8-bit (sign bit 7)."""
    q = np.asarray(q, np.float64)
    mags = _magnitudes(fmt)
    a = np.abs(q)
    # index of the largest grid value <= a (a >= 0 = mags[0])
    lo = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, mags.size - 1)
    hi = np.minimum(lo + 1, mags.size - 1)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= mags[-1], mags.size - 1, code)       # saturation
    sign_bit = 0x8 if fmt == "e2m1" else 0x80
    return (code | np.where(np.signbit(q), sign_bit, 0)).astype(np.uint8)


def format_values(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Values (float64) of element codes."""
    table = e2m1_table() if fmt == "e2m1" else e4m3_table()
    return table[np.asarray(codes, np.int64)]


def mx_quantize(v: np.ndarray, fmt: str):
    """Quantise values v [..., K] (float64, finite, K a multiple of 32) per
    32-value block along the last axis. Returns (codes uint8 [..., K],
    exponent bytes uint8 [..., K/32])."""
    v = np.asarray(v, np.float64)
    K = v.shape[-1]
    blocks = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - ACT_EMAX[fmt],
                     0.0)
    byte = np.clip(X + E8M0_BIAS, 0, 254).astype(np.int64)
    q = blocks / np.ldexp(1.0, byte - E8M0_BIAS)[..., None]    # exact: a power of two
    codes = round_to_format(q, fmt).reshape(v.shape)
    return codes, byte.astype(np.uint8)


def mx_dequant(codes: np.ndarray, exps: np.ndarray, fmt: str) -> np.ndarray:
    """Values of MX-quantised activations (inverse of the layout of
    mx_quantize), float64."""
    vals = format_values(codes, fmt)
    K = vals.shape[-1]
    scale = np.repeat(e8m0_scale(exps), 32, axis=-1).reshape(vals.shape[:-1] + (K,))
    return vals * scale


def act_values(v: np.ndarray, act: str) -> np.ndarray:
    """The activation values a routed GEMM consumes: v itself for bf16,
    else v quantised per the reading above and dequantised."""
    if act == "bf16":
        return np.asarray(v, np.float64)
    if act not in ACT_EMAX:
        raise ValueError(f"unknown activation format {act!r}")
    return mx_dequant(*mx_quantize(v, act), act)


# ----------------------------------------------------------------------------
# Experts
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def glu_ffn(xs: np.ndarray, gate: np.ndarray, up: np.ndarray, down: np.ndarray,
            act: str = "bf16"):
    """One expert on the rows xs [m][L] (float64 values).

    gate, up: [I][L]; down: [L][I] (float64 values).
    Returns (h_bits uint16 [m][I], y float64 [m][L]) with
    h = bf16(silu(a(xs) gate^T) * (a(xs) up^T)) and y = a(h) down^T, where a
    is the identity for bf16 activations and the quantisation of act_values
    otherwise.
    """
    xa = act_values(xs, act)
    g = xa @ gate.T
    u = xa @ up.T
    h_bits = bf16_from_f64(silu(g) * u)
    y = act_values(f64_from_bf16(h_bits), act) @ down.T
    return h_bits, y


def combine(y_routed: np.ndarray, w: np.ndarray, y_shared: Optional[np.ndarray]):
    """out[t] = sum_j w[t,j] y_routed[t,j] + sum_s y_shared[s,t], in that order.

    y_routed: [T][k][L] float64; w: [T][k] float32; y_shared: [S][T][L] or None.
    Returns (out float64 [T][L], out bf16 bits [T][L]).
    """
    T, k, L = y_routed.shape
    acc = np.zeros((T, L), np.float64)
    w64 = np.asarray(w, np.float32).astype(np.float64)
    for j in range(k):
        acc = acc + w64[:, j:j + 1] * y_routed[:, j, :]
    if y_shared is not None:
        for s in range(y_shared.shape[0]):
            acc = acc + y_shared[s]
    return acc, bf16_from_f64(acc)


def _expert_values(ex: Mapping[str, np.ndarray], L: int, I: int):
    gate = dequant_mxfp4(ex["gate_q"], ex["gate_s"], I, L)
    up = dequant_mxfp4(ex["up_q"], ex["up_s"], I, L)
    down = dequant_mxfp4(ex["down_q"], ex["down_s"], L, I)
    return gate, up, down


def _shared_outputs(x64: np.ndarray, shared: Mapping[str, np.ndarray]):
    sg, su, sd = shared["sh_gate"], shared["sh_up"], shared["sh_down"]
    S = sg.shape[0]
    ys = []
    for s in range(S):
        _, y = glu_ffn(x64, f64_from_bf16(sg[s]), f64_from_bf16(su[s]), f64_from_bf16(sd[s]))
        ys.append(y)
    if not ys:
        return None
    return np.stack(ys, axis=0)


def forward_tokens(x_bits: np.ndarray, idx: np.ndarray, w: np.ndarray,
                   get_expert: Callable[[int], Mapping[str, np.ndarray]],
                   shared: Mapping[str, np.ndarray], L: int, I: int,
                   tokens: Optional[Sequence[int]] = None, act: str = "bf16"):
    """Routed + shared FFN and combine for the listed tokens (all by default),
    given their routing (idx [T][k], w [T][k]).

    get_expert(e) returns expert e's codes and scales (the generator's layout).
    Experts are visited once each, serving every listed route that selects
    them. act: the routed experts' activation format (ACT_FORMATS); the
    shared experts stay bf16. Returns (out float64 [n][L], out bf16 bits
    [n][L]).
    """
    T, k = idx.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    n = toks.size
    x64 = f64_from_bf16(np.asarray(x_bits)[toks])
    sel = np.asarray(idx)[toks]
    y_routed = np.zeros((n, k, L), np.float64)
    for e in np.unique(sel):
        rows, slots = np.nonzero(sel == e)
        gate, up, down = _expert_values(get_expert(int(e)), L, I)
        _, y = glu_ffn(x64[rows], gate, up, down, act)
        y_routed[rows, slots] = y
    y_sh = _shared_outputs(x64, shared)
    return combine(y_routed, np.asarray(w)[toks], y_sh)


def forward(x_bits: np.ndarray, router_bits: Optional[np.ndarray],
            experts: Mapping[str, np.ndarray], shared: Mapping[str, np.ndarray],
            k: int, logits: Optional[np.ndarray] = None,
            act: str = "bf16") -> Dict[str, np.ndarray]:
    """The whole layer on every token.

    experts holds stacked [E][...] codes and scales; logits, when given, replace
    the router step; act is the routed experts' activation format. Returns
    every intermediate the layer exposes.
    """
    T, L = np.asarray(x_bits).shape
    E, I = experts["gate_q"].shape[0], experts["gate_q"].shape[1]
    if logits is None:
        logits = router_logits(x_bits, router_bits)
    logits = np.asarray(logits, np.float32)
    idx = topk_select(logits, k)
    w = softmax_selected(logits, idx)
    counts, offsets, perm, inv = permute_routes(idx, E)

    def get(e):
        return {key: experts[key][e] for key in
                ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}

    out64, out_bits = forward_tokens(x_bits, idx, w, get, shared, L, I, act=act)
    return {"logits": logits, "idx": idx, "w": w, "counts": counts,
            "offsets": offsets, "perm": perm, "inv": inv,
            "out64": out64, "out": out_bits}


# ----------------------------------------------------------------------------
# The MoE block around the layer: input step and tail
# ----------------------------------------------------------------------------
#
# TokenSpeed section 4.3 computes the three projections of the MoE input, the
# router scores, the routed experts' latent input (hidden -> latent) and the
# shared experts' gate/up values, as one matrix multiply over weights stored
# one after another, with the shared activation applied in its epilogue.
# Sections 4.2 and 6 describe the tail: the routed result (a 3584-wide latent
# vector) is RMS-normalised and projected up to the 7168-wide hidden width,
# then the shared experts' full-width output and the running residual are
# added; partials travel as BF16, reductions and normalisation use FP32
# internally.
#
# Readings (the pages fix neither layout nor epsilon):
#   W_in rows, in order: E router rows, L latent rows, then for each shared
#     expert s its gate and up rows interleaved in groups of 16 (rows
#     E + L + 2*Is*s + 32*j + c: gate row 16*j + c for c < 16, up row
#     16*j + c - 16 otherwise). h column s*Is + 16*j + c is
#     bf16(silu(g) * u) of that group.
#   logits = fp32(z_router); x = bf16(z_latent).
#   RMSNorm: n = bf16(r / sqrt(mean(r^2) + eps) * gamma), eps = 1e-6, in
#     exact arithmetic here (FP32 on the GPU), rounded once.
#   The shared experts' output is one BF16 partial, the sum over experts:
#     sh = bf16(h W_sd^T) with W_sd [H][S*Is] holding the experts' down
#     matrices side by side along K.
#   out = bf16(n W_up^T + sh + residual), rounded once.

RMS_EPS = 1e-6


def shared_gate_up_rows(E: int, L: int, S: int, Is: int):
    """Row indices into W_in of every shared expert's gate and up matrices:
    (gate [S][Is], up [S][Is]) under the interleaved reading above."""
    gate = np.empty((S, Is), np.int64)
    up = np.empty((S, Is), np.int64)
    for s in range(S):
        base = E + L + 2 * Is * s
        for i in range(Is):
            j, c = divmod(i, 16)
            gate[s, i] = base + 32 * j + c
            up[s, i] = base + 32 * j + 16 + c
    return gate, up


def moe_input(u_bits: np.ndarray, w_in_bits: np.ndarray, E: int, L: int, S: int,
              Is: int) -> Dict[str, np.ndarray]:
    """The MoE input step on hidden rows u (bf16 bits [T][H]) with the packed
    input weight W_in (bf16 bits [E + L + 2 S Is][H]).

    Returns logits float32 [T][E], x bf16 bits [T][L], h bf16 bits
    [T][S*Is] and z float64 [T][rows] (the exact product)."""
    u = f64_from_bf16(u_bits)
    w = f64_from_bf16(w_in_bits)
    assert w.shape[0] == E + L + 2 * S * Is, "W_in rows"
    z = u @ w.T
    logits = f32_round(z[:, :E]).astype(np.float32)
    x = bf16_from_f64(z[:, E:E + L])
    gate_rows, up_rows = shared_gate_up_rows(E, L, S, Is)
    T = u.shape[0]
    h = np.empty((T, S * Is), np.uint16)
    for s in range(S):
        g = z[:, gate_rows[s]]
        v = z[:, up_rows[s]]
        h[:, s * Is:(s + 1) * Is] = bf16_from_f64(silu(g) * v)
    return {"logits": logits, "x": x, "h": h, "z": z}


def rms_norm(r_bits: np.ndarray, gamma_bits: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """n = bf16(r / sqrt(mean(r^2) + eps) * gamma) per row of r (bf16 bits
    [T][L]); gamma bf16 bits [L]. Returns bf16 bits [T][L]."""
    r = f64_from_bf16(r_bits)
    gamma = f64_from_bf16(gamma_bits)
    ms = np.mean(r * r, axis=1, keepdims=True)
    return bf16_from_f64(r / np.sqrt(ms + eps) * gamma[None, :])


def moe_tail(routed_bits: np.ndarray, h_bits: np.ndarray, gamma_bits: np.ndarray,
             w_up_bits: np.ndarray, w_sd_bits: np.ndarray, residual_bits: np.ndarray,
             eps: float = RMS_EPS) -> Dict[str, np.ndarray]:
    """The MoE tail: routed latent result (bf16 bits [T][L]), shared
    activations h (bf16 bits [T][S*Is]), gamma [L], W_up [H][L],
    W_sd [H][S*Is], residual [T][H]. Returns n, sh (bf16 bits), out64
    (float64 [T][H]) and out (bf16 bits [T][H])."""
    n = rms_norm(routed_bits, gamma_bits, eps)
    sh = bf16_from_f64(f64_from_bf16(h_bits) @ f64_from_bf16(w_sd_bits).T)
    out64 = (f64_from_bf16(n) @ f64_from_bf16(w_up_bits).T + f64_from_bf16(sh)
             + f64_from_bf16(residual_bits))
    return {"n": n, "sh": sh, "out64": out64, "out": bf16_from_f64(out64)}


def block_forward(u_bits: np.ndarray, residual_bits: np.ndarray, w_in_bits: np.ndarray,
                  experts: Mapping[str, np.ndarray], gamma_bits: np.ndarray,
                  w_up_bits: np.ndarray, w_sd_bits: np.ndarray, E: int, L: int, S: int,
                  Is: int, k: int, logits: Optional[np.ndarray] = None,
                  act: str = "bf16") -> Dict[str, np.ndarray]:
    """Input step, the routed layer (no shared experts of its own: here they
    read the hidden input) and the tail. logits, when given, replace the
    input step's router scores for the routing (the GPU's own logits in the
    parity tests). Returns the intermediates of all three."""
    inp = moe_input(u_bits, w_in_bits, E, L, S, Is)
    lg = inp["logits"] if logits is None else np.asarray(logits, np.float32)
    Hd = u_bits.shape[1]
    no_shared = {"sh_gate": np.zeros((0, 0, L), np.uint16),
                 "sh_up": np.zeros((0, 0, L), np.uint16),
                 "sh_down": np.zeros((0, L, 0), np.uint16)}
    routed = forward(inp["x"], None, experts, no_shared, k, logits=lg, act=act)
    tail = moe_tail(routed["out"], inp["h"], gamma_bits, w_up_bits, w_sd_bits,
                    residual_bits)
    assert tail["out"].shape == (u_bits.shape[0], Hd)
    return {"input": inp, "routed": routed, "tail": tail, "out": tail["out"],
            "out64": tail["out64"]}

"""Helpers shared by the GPU tests: moving seeded inputs to the device, running
the HIP path through the binding, and the parity bounds."""
from __future__ import annotations

import sys
import time
from typing import Callable, Dict, Optional

import numpy as np

import oracle as O
from workloads import Workload

WEIGHT_KEYS = ("router_w", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
               "sh_gate", "sh_up", "sh_down")


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def upload(inp: Dict[str, np.ndarray], dev) -> Dict[str, object]:
    out = {}
    for k in WEIGHT_KEYS + ("x", "logits"):
        if k in inp:
            out[k] = to_dev(inp[k], dev)
    return out


def alloc_routing(d, dev) -> Dict[str, object]:
    import torch
    R = d.T * d.k
    return {
        "logits": torch.empty((d.T, d.E), dtype=torch.float32, device=dev),
        "topk_idx": torch.empty((d.T, d.k), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((d.T, d.k), dtype=torch.float32, device=dev),
        "counts": torch.empty((d.E,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((d.E + 1,), dtype=torch.int32, device=dev),
        "perm": torch.empty((R,), dtype=torch.int32, device=dev),
        "inv_perm": torch.empty((R,), dtype=torch.int32, device=dev),
    }


def pack_on_device(lm, d, dev_inp: Dict[str, object]) -> Dict[str, object]:
    """The routed experts of dev_inp repacked by lmoe_pack_weights."""
    import torch
    dev = dev_inp["x"].device
    pk = {k: torch.empty(n, dtype=torch.uint8, device=dev)
          for k, n in lm.packed_sizes(d).items()}
    lm.pack_weights(d, dev_inp, pk)
    return pk


def run_forward(lm, w: Workload, dev_inp: Dict[str, object], routing: Optional[dict] = None,
                packed: bool = False, path: Optional[int] = None, act: int = 0):
    """Run lmoe_forward (or, packed, lmoe_pack_weights then
    lmoe_forward_packed; or, with `path`, lmoe_forward_ex on that path);
    returns (out bf16 bits numpy, routing dict of numpy)."""
    import torch
    d = w.dims
    dev = dev_inp["x"].device
    if routing is None:
        routing = alloc_routing(d, dev)
    if w.logits_given:
        routing["logits"] = dev_inp["logits"]
    out = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    if packed:
        pk = pack_on_device(lm, d, dev_inp)
        lm.forward_packed(d, dev_inp["x"], {**dev_inp, **pk}, w.logits_given, routing, out, ws,
                          act=act)
    elif path is not None:
        lm.forward_ex(d, dev_inp["x"], dev_inp, w.logits_given, routing, out, ws, path=path)
    else:
        lm.forward(d, dev_inp["x"], dev_inp, w.logits_given, routing, out, ws)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in routing.items()}
    return out.cpu().numpy().view(np.uint16), res


def out_bound(ref64: np.ndarray, rms: Optional[float] = None) -> np.ndarray:
    """Element-wise bound for a bf16 output against the float64 reference:
    1e-2 * rms(ref) for the arithmetic, plus half a bf16 ulp for the final
    rounding to bf16 that the output format itself imposes."""
    if rms is None:
        rms = float(np.sqrt(np.mean(ref64 ** 2)))
    tol = 1e-2 * rms
    mag = np.maximum(np.abs(ref64) + tol, np.finfo(np.float64).tiny)
    e = np.floor(np.log2(mag)).astype(np.int64)
    return tol + np.ldexp(1.0, e - 8)


# Model of the kernels' fp32 evaluation of a GLU input, g = sum_l x_l W_l over
# K values: |g_fp32 - g| <= H_ACC * 2^-24 * sum_l |x_l W_l|. The kernels add
# K/32 exact block sums into an fp32 accumulator; on the workloads that
# ordering stays below 4 * 2^-24 * sum |x W| (fp32 emulation on the host), so
# 16 leaves a margin of four. A larger H_ACC widens the allowance below, a
# smaller one can only make the check stricter.
H_ACC = 16.0
# The FP8 (E4M3) x FP4 scaled MFMA does not sum its products to fp32
# accuracy: on random operands (40 x 2048 outputs of 512 products each,
# in-bounds probe on gfx950) its error reached 392 * 2^-24 * sum |a b|, while
# FP4 x FP4 sums were exact. The quantised-activation tests model g and u of
# the E4M3 path with four times that.
H_ACC_E4M3 = 1600.0


def h_flip_allowance(x64: np.ndarray, gate: np.ndarray, up: np.ndarray, down: np.ndarray,
                     act: str = "bf16"):
    """Allowance for one expert's GLU, per row of x64 and output column:
    where fp32 g and u may round h = bf16(silu(g) u) to the other side of a
    bf16 rounding midpoint than the float64 oracle does, the two h differ by
    one bf16 ulp, and output l moves by that ulp times |down[l, i]|. An h
    element is counted when the distance of the float64 silu(g) u to its
    nearest rounding midpoint is at most the propagated evaluation error
    (H_ACC model for g and u, 8 fp32 ulp for silu and the product); each
    counted element adds twice its bf16 spacing (covering the spacing change
    at a power of two) times |down[l, i]|. With quantised activations (act
    E4M3 / E2M1) the GLU reads the quantised x, and a flipped h may also move
    its quantised value by one step of the element grid (times the block
    scale), which is added for the counted elements. Returns [rows][L]."""
    xa = O.act_values(x64, act)
    g = xa @ gate.T
    u = xa @ up.T
    ax = np.abs(xa)
    hacc = H_ACC_E4M3 if act == "e4m3" else H_ACC
    dg = hacc * 2.0 ** -24 * (ax @ np.abs(gate).T)
    du = hacc * 2.0 ** -24 * (ax @ np.abs(up).T)
    with np.errstate(over="ignore", invalid="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
        s = g * sig
        ds_dg = sig * (1.0 + g * (1.0 - sig))
    v = s * u
    dv = np.abs(ds_dg * u) * dg + np.abs(s) * du + 8 * 2.0 ** -24 * np.abs(v)
    h = O.f64_from_bf16(O.bf16_from_f64(v))
    av = np.abs(v)
    e = np.floor(np.log2(np.where(av > 0, av, 1.0)))
    half = np.ldexp(1.0, (e - 8).astype(np.int64))       # half the bf16 spacing at |v|
    near = (av > 0) & (np.abs(np.abs(v - h) - half) <= dv)
    flip = np.where(near, 4.0 * half, 0.0)               # twice the spacing
    if act != "bf16" and near.any():
        codes, exps = O.mx_quantize(h, act)
        scale = np.repeat(O.e8m0_scale(exps), 32, axis=-1).reshape(h.shape)
        mags = np.unique(np.abs(O.format_values(np.arange(16 if act == "e2m1" else 127), act)))
        k = np.clip(np.searchsorted(mags, np.abs(h) / scale), 1, mags.size - 1)
        step = np.maximum(mags[k] - mags[k - 1], mags[np.minimum(k + 1, mags.size - 1)] - mags[k])
        flip = flip + np.where(near, step * scale, 0.0)
        # a flipped block maximum can move the block's scale exponent by one,
        # which requantises all 32 values of the block: each may then move by
        # a step of the grid at twice the scale
        blk = np.abs(h).reshape(h.shape[:-1] + (-1, 32))
        top = (blk == blk.max(axis=-1, keepdims=True)) & near.reshape(blk.shape)
        moved = np.repeat(top.any(axis=-1), 32, axis=-1).reshape(h.shape)
        flip = flip + np.where(moved, 2.0 * step * scale, 0.0)
    return flip @ np.abs(down).T


def flip_allowance_fn(x_bits: np.ndarray, idx: np.ndarray, w: np.ndarray,
                      get_expert: Callable[[int], Dict[str, np.ndarray]],
                      shared: Optional[Dict[str, np.ndarray]], L: int, I: int,
                      experts: Optional[set] = None, act: str = "bf16"):
    """fn(rows) -> [len(rows)][L]: the h-rounding allowance of those rows of
    x (h_flip_allowance of each selected expert, weighted by the token's
    softmax weight as in the combine, plus each shared expert with weight 1).
    `experts` restricts the routed experts counted (the others contribute
    nothing, e.g. silenced experts)."""
    def fn(rows):
        rows = np.asarray(rows, np.int64)
        x64 = O.f64_from_bf16(np.asarray(x_bits)[rows])
        sel = np.asarray(idx)[rows]
        acc = np.zeros((rows.size, L), np.float64)
        for e in np.unique(sel):
            if experts is not None and int(e) not in experts:
                continue
            rr, jj = np.nonzero(sel == e)
            ex = get_expert(int(e))
            gate = O.dequant_mxfp4(ex["gate_q"], ex["gate_s"], I, L)
            up = O.dequant_mxfp4(ex["up_q"], ex["up_s"], I, L)
            down = O.dequant_mxfp4(ex["down_q"], ex["down_s"], L, I)
            a = h_flip_allowance(x64[rr], gate, up, down, act)
            acc[rr] += np.asarray(w, np.float64)[rows[rr], jj][:, None] * a
        if shared is not None:
            for sidx in range(shared["sh_gate"].shape[0]):
                acc += h_flip_allowance(x64, O.f64_from_bf16(shared["sh_gate"][sidx]),
                                        O.f64_from_bf16(shared["sh_up"][sidx]),
                                        O.f64_from_bf16(shared["sh_down"][sidx]))
        return acc
    return fn


def check_out(got_bits: np.ndarray, ref64: np.ndarray, what: str, rms: Optional[float] = None,
              allowance_fn=None, rows: Optional[np.ndarray] = None):
    """Outputs [n][L] within out_bound of the float64 reference. Where that
    fails and `allowance_fn` is given, the failing rows are checked again with
    their h-rounding allowance added (allowance_fn(token ids) with the token
    ids `rows` of the compared rows, default 0..n-1)."""
    got = O.f64_from_bf16(got_bits)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref64 ** 2)))
    bound = out_bound(ref64, rms)
    err = np.abs(got - ref64)
    n_flip = 0
    if allowance_fn is not None and not np.all(err <= bound):
        fail = np.nonzero(np.any(~(err <= bound), axis=1))[0]
        tok = (np.arange(got.shape[0]) if rows is None else np.asarray(rows))[fail]
        n_flip = int(np.sum(~(err[fail] <= bound[fail])))
        bound = bound.copy()
        bound[fail] += allowance_fn(tok)
    bad = np.nonzero(~(err <= bound))
    rel_rms = float(np.sqrt(np.mean((got - ref64) ** 2)) / rms)
    log(f"{what}: max|err|/rms={err.max() / rms:.3e} rms(err)/rms={rel_rms:.3e}"
        + (f"; {n_flip} of {err.size} outputs within the h-rounding allowance only"
           if n_flip else ""))
    assert bad[0].size == 0, (
        f"{what}: {bad[0].size} outputs out of bound; first at {tuple(b[0] for b in bad)}: "
        f"got {got[bad][0]!r} ref {ref64[bad][0]!r} bound {bound[bad][0]!r}")
    # the pages report stage RMS relative errors around 1e-3; bf16 output
    # rounding alone contributes ~1.1e-3
    assert rel_rms < 3e-3, f"{what}: rms error {rel_rms:.3e}"


def logits_bound(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """Worst-case fp32 summation bound on |gpu_logit - oracle_logit| per (t, e):
    (L + 2) * 2^-24 * sum_l |x w| plus the final rounding of the oracle."""
    ax = np.abs(O.f64_from_bf16(x_bits))
    aw = np.abs(O.f64_from_bf16(wr_bits))
    L = ax.shape[1]
    s = ax @ aw.T
    return (L + 2) * 2.0 ** -24 * s + 2.0 ** -24 * s


def topk_w_bound(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Bound on |w_gpu - w_oracle| for the softmax over the selected logits,
    per selected route, for the kernels' evaluation: d_j = fl(l_j - l_0) in
    fp32, z_j = expf(d_j), s = fp32 sum of the k terms in some order,
    w_j = z_j / s correctly rounded. With u = 2^-24 (half an fp32 ulp) and an
    expf error of at most 2 ulp (<= 8u relative), to first order:
      rounding of d_j, carried through exp      |d_j| u
      expf                                      8u
      the same two in every term of s           max_i |d_i| u + 8u
      summing k positive terms                  (k - 1) u
      the division, the oracle's own rounding   2u
    so |w_gpu - w_ref| <= (|d_j| + max_i |d_i| + k + 17) u w_ref, and 1% more
    for second-order terms."""
    lg = np.asarray(logits, np.float32).astype(np.float64)
    sel = np.take_along_axis(lg, np.asarray(idx, np.int64), axis=1)
    with np.errstate(invalid="ignore"):
        d = np.abs(sel - sel[:, :1])
        w = O.softmax_selected(logits, idx).astype(np.float64)
    # a -inf logit below a finite first one has weight exactly 0 on both
    # sides (expf(-inf) = 0): bound 0 there; rows with NaN weights are not
    # compared
    fin = np.isfinite(d)
    d = np.where(fin, d, 0.0)
    k = sel.shape[1]
    rel = (d + d.max(axis=1, keepdims=True) + k + 17) * 2.0 ** -24 * 1.01
    return np.where(fin, rel * np.abs(np.nan_to_num(w)), 0.0)


def check_routing_exact(res: Dict[str, np.ndarray], logits: np.ndarray, k: int, what: str):
    """The routing outputs of one call against the oracle's routing steps on
    the same logits (given logits, or the GPU's own computed ones): indices,
    counts, offsets, perm and inv_perm bit for bit; weights within
    topk_w_bound. Returns the largest weight error in fp32 ulps."""
    E = logits.shape[1]
    idx = O.topk_select(logits, k)
    with np.errstate(invalid="ignore"):
        w = O.softmax_selected(logits, idx)
    counts, offsets, perm, inv = O.permute_routes(idx, E)
    bad = np.nonzero(np.any(res["topk_idx"] != idx, axis=1))[0]
    assert bad.size == 0, (f"{what}: top-k indices differ on {bad.size} tokens, first {bad[0]}: "
                           f"got {res['topk_idx'][bad[0]].tolist()} want {idx[bad[0]].tolist()}")
    fin = np.isfinite(w)
    err = np.abs(res["topk_w"].astype(np.float64) - w.astype(np.float64))
    bound = topk_w_bound(logits, idx)
    assert np.all(err[fin] <= bound[fin]), f"{what}: weights differ beyond the bound"
    ulp = np.spacing(np.abs(w[fin]).astype(np.float32)).astype(np.float64)
    max_ulp = float((err[fin] / ulp).max()) if fin.any() else 0.0
    assert np.array_equal(res["counts"], counts), f"{what}: counts differ"
    assert np.array_equal(res["offsets"], offsets), f"{what}: offsets differ"
    assert np.array_equal(res["perm"], perm), f"{what}: perm differs"
    assert np.array_equal(res["inv_perm"], inv), f"{what}: inv_perm differs"
    log(f"{what}: routing bit-exact ({logits.shape[0]} tokens, E={E}, k={k}); "
        f"weights within {max_ulp:.1f} ulp")
    return max_ulp


def check_routing_against_oracle(gpu_idx: np.ndarray, gpu_logits: np.ndarray,
                                 ref_logits: np.ndarray, bound: np.ndarray, k: int, what: str):
    """GPU logits within the summation bound; the GPU's selected set equals the
    oracle's wherever the oracle's top-k boundary gap exceeds twice the bound,
    and elsewhere every GPU choice is a valid top-k choice within the bound.
    Returns the boolean mask of tokens whose sets agree."""
    g64, r64 = gpu_logits.astype(np.float64), ref_logits.astype(np.float64)
    both_nan = np.isnan(g64) & np.isnan(r64)
    d = np.where(both_nan, 0.0, np.abs(g64 - r64))
    assert np.all(d <= bound), f"{what}: logits off by {np.nanmax(d - bound):.3e} beyond bound"
    ref_idx = O.topk_select(ref_logits, k)
    same = np.array([set(a) == set(b) for a, b in zip(gpu_idx.tolist(), ref_idx.tolist())])
    lg = ref_logits.astype(np.float64)
    srt = -np.sort(-np.nan_to_num(lg, nan=-np.inf), axis=1)
    for t in np.nonzero(~same)[0]:
        tb = bound[t].max()
        gap = srt[t, k - 1] - srt[t, k] if lg.shape[1] > k else np.inf
        assert gap <= 2 * tb, f"{what}: token {t} routed differently with a clear gap {gap:.3e}"
        kth = srt[t, k - 1]
        assert np.all(lg[t, gpu_idx[t]] >= kth - 2 * tb), f"{what}: token {t} invalid choice"
    log(f"{what}: routing sets agree on {same.sum()}/{same.size} tokens")
    return same

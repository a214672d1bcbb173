"""Python binding of liblmoe.so, the LatentMoE MXFP4 (w4a16) layer for MI355X.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch supplies device memory and the current stream. The library is
loaded from this package directory; importing the binding when it is missing
raises, there is no fallback of any kind.

Functions mirror the C ABI in include/lmoe.h:
  workspace_bytes(dims)
  route(dims, x, router_w, logits_given, routing, ws)
  forward(dims, x, weights, logits_given, routing, out, ws)
  forward_ex(dims, x, weights, logits_given, routing, out, ws, side_stream, fork_event,
             join_event)
  wait_errors(ws, count)
  forward_noalloc(dims, x, weights, logits_given, routing, out)
  packed_sizes(dims)
  pack_weights(dims, weights, packed)
  forward_packed(dims, x, weights, logits_given, routing, out, ws, side_stream, fork_event,
                 join_event)
  debug_dequant_mxfp4(q, s, rows, K, out)
  status_string(code)
  block_workspace_bytes(bdims)
  moe_input(bdims, u, w_in, logits, x, h_sh, ws)
  moe_tail(bdims, routed, h_sh, norm_w, w_up, w_sd, residual, out, ws)
  block_forward(bdims, u, residual, block_weights, experts, routing, out, ws)
`dims` is a Dims-like object (attributes T, L, E, k, I, S, Is) or a tuple in
that order, `bdims` likewise with attributes T, H, L, E, k, I, S, Is; tensors are torch CUDA tensors (bf16 data may be torch.bfloat16,
torch.int16 or torch.uint16 views), `weights` and `routing` are dicts keyed by
the C struct member names.
"""
from __future__ import annotations

import ctypes
import os
from typing import Mapping, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblmoe.so")

LMOE_OK = 0
LMOE_ERR_NULL = 1
LMOE_ERR_SHAPE = 2
LMOE_ERR_ALIGN = 3
LMOE_ERR_WORKSPACE = 4
LMOE_ERR_HIP = 5
# scratch of lmoe_forward_noalloc per GPU (LMOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
# the decode kernels' counter block at the start of a workspace (LMOE_COUNTER_BYTES)
COUNTER_BYTES = 256 << 10

EXPORTS = ("lmoe_workspace_bytes", "lmoe_route", "lmoe_forward", "lmoe_forward_ex",
           "lmoe_forward_traced", "lmoe_wait_errors", "lmoe_forward_noalloc", "lmoe_stage_name", "lmoe_path_name",
           "lmoe_debug_dequant_mxfp4", "lmoe_status_string", "lmoe_packed_sizes_of",
           "lmoe_pack_weights", "lmoe_forward_packed", "lmoe_debug_read_stream", "lmoe_debug_mfma_rate",
           "lmoe_debug_quantize_act", "lmoe_block_workspace_bytes", "lmoe_moe_input",
           "lmoe_moe_tail", "lmoe_block_forward")
# members of lmoe_packed_sizes / the packed routed-expert arrays
PACKED_KEYS = ("gu_q", "gu_s", "down_q", "down_s")

# Stage boundaries recorded by forward_traced (LMOE_STAGE_* in lmoe.h).
STAGES = ("begin", "router", "topk", "permute", "gate_up", "down", "shared_gate_up",
          "shared_down", "combine")
NUM_STAGE_EVENTS = len(STAGES)


class lmoe_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "L", "E", "k", "I", "S", "Is")]


class lmoe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
        "sh_gate", "sh_up", "sh_down")]


class lmoe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm")]


class lmoe_exec(ctypes.Structure):
    _fields_ = [("side_stream", ctypes.c_void_p), ("fork_event", ctypes.c_void_p),
                ("join_event", ctypes.c_void_p), ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                ("path", ctypes.c_int32), ("act_format", ctypes.c_int32)]


# lmoe_exec.path
PATH_AUTO, PATH_GROUPED, PATH_FUSED = 0, 1, 2
# lmoe_exec.act_format
ACT_BF16, ACT_E4M3, ACT_E2M1 = 0, 1, 2


def _exec(side_stream, fork_event, join_event, stage_events, path=PATH_AUTO, act=ACT_BF16):
    if side_stream is None and stage_events is None and path == PATH_AUTO and act == ACT_BF16:
        return None
    ex = lmoe_exec(side_stream and int(side_stream), fork_event and int(fork_event),
                   join_event and int(join_event), None, int(path), int(act))
    if stage_events is not None:
        if len(stage_events) != NUM_STAGE_EVENTS:
            raise ValueError(f"need {NUM_STAGE_EVENTS} events")
        arr = (ctypes.c_void_p * NUM_STAGE_EVENTS)(*[int(e) for e in stage_events])
        ex.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        ex._keep = arr
    return ex


class lmoe_block_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "L", "E", "k", "I", "S", "Is")]


class lmoe_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_in", "norm_w", "w_up", "w_sd")]


class lmoe_packed_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("gu_q", "gu_s", "down_q", "down_s")]


class lmoe_packed_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "gu_q", "gu_s", "down_q", "down_s", "sh_gate", "sh_up", "sh_down")]


class LmoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: status {code} ({msg})")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python mxfp4_latent_mixture_amd/build.py` "
            "(hipcc, gfx950). There is no CPU fallback.")
    # torch ships its own HIP runtime under the same soname as the system's:
    # loading torch first makes this library bind to the runtime that
    # allocates the tensors it is handed (one runtime per process)
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    dp = ctypes.POINTER(lmoe_dims)
    lib.lmoe_workspace_bytes.argtypes = [dp]
    lib.lmoe_workspace_bytes.restype = sz
    lib.lmoe_route.argtypes = [dp, vp, vp, ctypes.c_int, ctypes.POINTER(lmoe_routing), vp, sz, vp]
    lib.lmoe_route.restype = ctypes.c_int
    lib.lmoe_forward.argtypes = [dp, vp, ctypes.POINTER(lmoe_weights), ctypes.c_int,
                                 ctypes.POINTER(lmoe_routing), vp, vp, sz, vp]
    lib.lmoe_forward.restype = ctypes.c_int
    lib.lmoe_forward_ex.argtypes = [dp, vp, ctypes.POINTER(lmoe_weights), ctypes.c_int,
                                    ctypes.POINTER(lmoe_routing), vp, vp, sz, vp,
                                    ctypes.POINTER(lmoe_exec)]
    lib.lmoe_forward_ex.restype = ctypes.c_int
    lib.lmoe_forward_noalloc.argtypes = [dp, vp, ctypes.POINTER(lmoe_weights), ctypes.c_int,
                                         ctypes.POINTER(lmoe_routing), vp, vp]
    lib.lmoe_forward_noalloc.restype = ctypes.c_int
    lib.lmoe_packed_sizes_of.argtypes = [dp, ctypes.POINTER(lmoe_packed_sizes)]
    lib.lmoe_packed_sizes_of.restype = ctypes.c_int
    lib.lmoe_pack_weights.argtypes = [dp, ctypes.POINTER(lmoe_weights), vp, vp, vp, vp, vp]
    lib.lmoe_pack_weights.restype = ctypes.c_int
    lib.lmoe_forward_packed.argtypes = [dp, vp, ctypes.POINTER(lmoe_packed_weights), ctypes.c_int,
                                        ctypes.POINTER(lmoe_routing), vp, vp, sz, vp,
                                        ctypes.POINTER(lmoe_exec)]
    lib.lmoe_forward_packed.restype = ctypes.c_int
    lib.lmoe_wait_errors.argtypes = [vp, sz, vp, vp]
    lib.lmoe_wait_errors.restype = ctypes.c_int
    lib.lmoe_forward_traced.argtypes = [dp, vp, ctypes.POINTER(lmoe_weights), ctypes.c_int,
                                        ctypes.POINTER(lmoe_routing), vp, vp, sz, vp,
                                        ctypes.POINTER(vp)]
    lib.lmoe_forward_traced.restype = ctypes.c_int
    lib.lmoe_path_name.argtypes = [dp, ctypes.c_int]
    lib.lmoe_path_name.restype = ctypes.c_char_p
    lib.lmoe_stage_name.argtypes = [ctypes.c_int]
    lib.lmoe_stage_name.restype = ctypes.c_char_p
    lib.lmoe_debug_quantize_act.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            vp, vp, vp]
    lib.lmoe_debug_quantize_act.restype = ctypes.c_int
    lib.lmoe_debug_read_stream.argtypes = [vp, sz, vp, i32, vp]
    lib.lmoe_debug_read_stream.restype = ctypes.c_int
    lib.lmoe_debug_mfma_rate.argtypes = [i32, vp, i32, vp]
    lib.lmoe_debug_mfma_rate.restype = ctypes.c_int
    lib.lmoe_debug_dequant_mxfp4.argtypes = [vp, vp, i32, i32, vp, vp]
    lib.lmoe_debug_dequant_mxfp4.restype = ctypes.c_int
    bdp = ctypes.POINTER(lmoe_block_dims)
    lib.lmoe_block_workspace_bytes.argtypes = [bdp]
    lib.lmoe_block_workspace_bytes.restype = sz
    lib.lmoe_moe_input.argtypes = [bdp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lmoe_moe_input.restype = ctypes.c_int
    lib.lmoe_moe_tail.argtypes = [bdp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lmoe_moe_tail.restype = ctypes.c_int
    lib.lmoe_block_forward.argtypes = [bdp, vp, vp, ctypes.POINTER(lmoe_block_weights),
                                       ctypes.POINTER(lmoe_weights),
                                       ctypes.POINTER(lmoe_routing), vp, vp, sz, vp]
    lib.lmoe_block_forward.restype = ctypes.c_int
    lib.lmoe_status_string.argtypes = [ctypes.c_int]
    lib.lmoe_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def status_string(code: int) -> str:
    return _lib.lmoe_status_string(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != LMOE_OK:
        raise LmoeError(fn, code, status_string(code))


def _dims(d) -> lmoe_dims:
    if isinstance(d, lmoe_dims):
        return d
    if isinstance(d, (tuple, list)):
        return lmoe_dims(*[int(v) for v in d])
    return lmoe_dims(int(d.T), int(d.L), int(d.E), int(d.k), int(d.I), int(d.S), int(d.Is))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _routing(r: Optional[Mapping]) -> Optional[lmoe_routing]:
    if r is None:
        return None
    return lmoe_routing(*[_ptr(r.get(n)) for n, _ in lmoe_routing._fields_])


def _weights(w: Mapping) -> lmoe_weights:
    return lmoe_weights(*[_ptr(w.get(n)) for n, _ in lmoe_weights._fields_])


def workspace_bytes(dims) -> int:
    d = _dims(dims)
    return int(_lib.lmoe_workspace_bytes(ctypes.byref(d)))


def route(dims, x, router_w, logits_given: bool, routing: Optional[Mapping], ws,
          stream=None) -> None:
    d = _dims(dims)
    r = _routing(routing)
    code = _lib.lmoe_route(ctypes.byref(d), _ptr(x), _ptr(router_w), int(bool(logits_given)),
                           ctypes.byref(r) if r is not None else None, _ptr(ws),
                           ws.numel() * ws.element_size() if ws is not None else 0,
                           _stream(stream))
    _check("lmoe_route", code)


def forward(dims, x, weights: Mapping, logits_given: bool, routing: Optional[Mapping], out, ws,
            stream=None) -> None:
    d = _dims(dims)
    r = _routing(routing)
    w = _weights(weights)
    code = _lib.lmoe_forward(ctypes.byref(d), _ptr(x), ctypes.byref(w), int(bool(logits_given)),
                             ctypes.byref(r) if r is not None else None, _ptr(out), _ptr(ws),
                             ws.numel() * ws.element_size() if ws is not None else 0,
                             _stream(stream))
    _check("lmoe_forward", code)


def forward_ex(dims, x, weights: Mapping, logits_given: bool, routing: Optional[Mapping], out,
               ws, side_stream=None, fork_event=None, join_event=None, stream=None,
               stage_events=None, path=PATH_AUTO, act=ACT_BF16) -> None:
    """forward() with the shared experts on the caller's side_stream (an int
    hipStream_t), forked and joined by the caller's fork_event / join_event
    (int hipEvent_t); side_stream None runs every stage on `stream`.
    stage_events: NUM_STAGE_EVENTS hipEvent_t recorded at the stage
    boundaries (every stage on `stream`). path: PATH_AUTO, PATH_GROUPED or
    PATH_FUSED (lmoe_exec.path)."""
    d = _dims(dims)
    r = _routing(routing)
    w = _weights(weights)
    ex = _exec(side_stream, fork_event, join_event, stage_events, path, act)
    code = _lib.lmoe_forward_ex(ctypes.byref(d), _ptr(x), ctypes.byref(w),
                                int(bool(logits_given)),
                                ctypes.byref(r) if r is not None else None, _ptr(out), _ptr(ws),
                                ws.numel() * ws.element_size() if ws is not None else 0,
                                _stream(stream), ctypes.byref(ex) if ex is not None else None)
    _check("lmoe_forward_ex", code)


def forward_noalloc(dims, x, weights: Mapping, logits_given: bool, routing: Optional[Mapping],
                    out, stream=None) -> None:
    """forward() with the library's static per-GPU scratch as workspace: no
    device allocation; calls that overlap on one GPU race."""
    d = _dims(dims)
    r = _routing(routing)
    w = _weights(weights)
    code = _lib.lmoe_forward_noalloc(ctypes.byref(d), _ptr(x), ctypes.byref(w),
                                     int(bool(logits_given)),
                                     ctypes.byref(r) if r is not None else None, _ptr(out),
                                     _stream(stream))
    _check("lmoe_forward_noalloc", code)


def packed_sizes(dims) -> dict:
    """Bytes of each tile-packed routed-expert array (PACKED_KEYS)."""
    d = _dims(dims)
    z = lmoe_packed_sizes()
    _check("lmoe_packed_sizes_of", _lib.lmoe_packed_sizes_of(ctypes.byref(d), ctypes.byref(z)))
    return {k: int(getattr(z, k)) for k in PACKED_KEYS}


def pack_weights(dims, weights: Mapping, packed: Mapping, stream=None) -> None:
    """Repack the routed experts of `weights` (row-major) into the uint8
    device tensors packed[k] for k in PACKED_KEYS (packed_sizes bytes)."""
    d = _dims(dims)
    w = _weights(weights)
    code = _lib.lmoe_pack_weights(ctypes.byref(d), ctypes.byref(w),
                                  *[_ptr(packed[k]) for k in PACKED_KEYS], _stream(stream))
    _check("lmoe_pack_weights", code)


def forward_packed(dims, x, weights: Mapping, logits_given: bool, routing: Optional[Mapping],
                   out, ws, side_stream=None, fork_event=None, join_event=None,
                   stream=None, stage_events=None, act=ACT_BF16) -> None:
    """forward_ex() on tile-packed routed experts: `weights` holds router_w,
    the PACKED_KEYS arrays and the shared-expert tensors. act: the routed
    experts' activation format (ACT_BF16, ACT_E4M3, ACT_E2M1)."""
    d = _dims(dims)
    r = _routing(routing)
    w = lmoe_packed_weights(*[_ptr(weights.get(n)) for n, _ in lmoe_packed_weights._fields_])
    ex = _exec(side_stream, fork_event, join_event, stage_events, act=act)
    code = _lib.lmoe_forward_packed(ctypes.byref(d), _ptr(x), ctypes.byref(w),
                                    int(bool(logits_given)),
                                    ctypes.byref(r) if r is not None else None, _ptr(out),
                                    _ptr(ws), ws.numel() * ws.element_size() if ws is not None
                                    else 0, _stream(stream),
                                    ctypes.byref(ex) if ex is not None else None)
    _check("lmoe_forward_packed", code)


def wait_errors(ws, count, stream=None) -> None:
    """Enqueue a copy of the workspace's abandoned-wait count into the int32
    device tensor `count` and reset it."""
    code = _lib.lmoe_wait_errors(_ptr(ws), ws.numel() * ws.element_size() if ws is not None
                                 else 0, _ptr(count), _stream(stream))
    _check("lmoe_wait_errors", code)


def forward_traced(dims, x, weights: Mapping, logits_given: bool, routing: Optional[Mapping], out,
                   ws, events, stream=None) -> None:
    """forward() that also records NUM_STAGE_EVENTS caller-created hipEvent_t
    handles (ints) at the stage boundaries listed in STAGES."""
    d = _dims(dims)
    r = _routing(routing)
    w = _weights(weights)
    if len(events) != NUM_STAGE_EVENTS:
        raise ValueError(f"need {NUM_STAGE_EVENTS} events")
    ev = (ctypes.c_void_p * NUM_STAGE_EVENTS)(*[int(e) for e in events])
    code = _lib.lmoe_forward_traced(ctypes.byref(d), _ptr(x), ctypes.byref(w),
                                    int(bool(logits_given)),
                                    ctypes.byref(r) if r is not None else None, _ptr(out),
                                    _ptr(ws), ws.numel() * ws.element_size() if ws is not None
                                    else 0, _stream(stream), ev)
    _check("lmoe_forward_traced", code)


def path_name(dims, logits_given: bool = False) -> str:
    d = _dims(dims)
    return _lib.lmoe_path_name(ctypes.byref(d), int(bool(logits_given))).decode()


def stage_name(i: int) -> str:
    return _lib.lmoe_stage_name(int(i)).decode()


def debug_mfma_rate(iters: int, sink, blocks: int, stream=None) -> None:
    """`blocks` workgroups of four waves each issue iters * 8 bf16 32x32x16
    MFMAs on register operands (the sustained MFMA rate); one word per
    workgroup lands in the int32 device tensor sink."""
    code = _lib.lmoe_debug_mfma_rate(int(iters), _ptr(sink), int(blocks), _stream(stream))
    _check("lmoe_debug_mfma_rate", code)


def debug_read_stream(buf, sink, blocks: int, stream=None) -> None:
    """Read every byte of the device tensor buf once (the plain HBM read
    rate); one word per workgroup lands in the int32 device tensor sink."""
    code = _lib.lmoe_debug_read_stream(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                       int(blocks), _stream(stream))
    _check("lmoe_debug_read_stream", code)


def debug_quantize_act(src, rows: int, K: int, act: int, codes, exps, stream=None) -> None:
    """Quantise a bf16 [rows][K] device tensor with the device routine of the
    quantised activation path (act ACT_E4M3 or ACT_E2M1) into codes and
    exponent bytes (lmoe_debug_quantize_act)."""
    code = _lib.lmoe_debug_quantize_act(_ptr(src), int(rows), int(K), int(act), _ptr(codes),
                                        _ptr(exps), _stream(stream))
    _check("lmoe_debug_quantize_act", code)


def debug_dequant_mxfp4(q, s, rows: int, K: int, out, stream=None) -> None:
    code = _lib.lmoe_debug_dequant_mxfp4(_ptr(q), _ptr(s), int(rows), int(K), _ptr(out),
                                         _stream(stream))
    _check("lmoe_debug_dequant_mxfp4", code)


def _bdims(d) -> lmoe_block_dims:
    if isinstance(d, lmoe_block_dims):
        return d
    if isinstance(d, (tuple, list)):
        return lmoe_block_dims(*[int(v) for v in d])
    return lmoe_block_dims(int(d.T), int(d.H), int(d.L), int(d.E), int(d.k), int(d.I),
                           int(d.S), int(d.Is))


def _nbytes(t) -> int:
    return t.numel() * t.element_size() if t is not None else 0


def block_workspace_bytes(bdims) -> int:
    d = _bdims(bdims)
    return int(_lib.lmoe_block_workspace_bytes(ctypes.byref(d)))


def moe_input(bdims, u, w_in, logits, x, h_sh, ws, stream=None) -> None:
    """The MoE input step (lmoe_moe_input): router scores, latent rows and
    the shared experts' activations from one packed projection of u."""
    d = _bdims(bdims)
    code = _lib.lmoe_moe_input(ctypes.byref(d), _ptr(u), _ptr(w_in), _ptr(logits), _ptr(x),
                               _ptr(h_sh), _ptr(ws), _nbytes(ws), _stream(stream))
    _check("lmoe_moe_input", code)


def moe_tail(bdims, routed, h_sh, norm_w, w_up, w_sd, residual, out, ws, stream=None) -> None:
    """The MoE tail (lmoe_moe_tail): RMSNorm of the routed result, the
    up-projection, plus the shared output and the residual."""
    d = _bdims(bdims)
    code = _lib.lmoe_moe_tail(ctypes.byref(d), _ptr(routed), _ptr(h_sh), _ptr(norm_w),
                              _ptr(w_up), _ptr(w_sd), _ptr(residual), _ptr(out), _ptr(ws),
                              _nbytes(ws), _stream(stream))
    _check("lmoe_moe_tail", code)


def block_forward(bdims, u, residual, block_weights: Mapping, experts: Mapping,
                  routing: Optional[Mapping], out, ws, stream=None) -> None:
    """The whole MoE block (lmoe_block_forward): block_weights holds w_in,
    norm_w, w_up, w_sd; experts the routed MXFP4 arrays (lmoe_weights keys)."""
    d = _bdims(bdims)
    bw = lmoe_block_weights(*[_ptr(block_weights.get(n)) for n, _ in lmoe_block_weights._fields_])
    w = _weights(experts)
    r = _routing(routing)
    code = _lib.lmoe_block_forward(ctypes.byref(d), _ptr(u), _ptr(residual), ctypes.byref(bw),
                                   ctypes.byref(w), ctypes.byref(r) if r is not None else None,
                                   _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))
    _check("lmoe_block_forward", code)

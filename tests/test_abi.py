"""CPU checks of the C ABI: the library loads, exports every declared entry
point, sizes its workspace, and rejects bad arguments on the host before any
launch (every call below fails validation, so no kernel is ever enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmoe.h")


@pytest.fixture(scope="module")
def lm():
    import mxfp4_latent_mixture_amd as lm
    return lm


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmoe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    assert names == sorted(["lmoe_workspace_bytes", "lmoe_route", "lmoe_forward",
                            "lmoe_forward_ex", "lmoe_forward_traced", "lmoe_wait_errors",
                            "lmoe_forward_noalloc", "lmoe_packed_sizes_of",
                            "lmoe_pack_weights", "lmoe_forward_packed",
                            "lmoe_debug_read_stream", "lmoe_debug_mfma_rate", "lmoe_debug_quantize_act",
                            "lmoe_stage_name", "lmoe_path_name",
                            "lmoe_debug_dequant_mxfp4", "lmoe_status_string",
                            "lmoe_block_workspace_bytes", "lmoe_moe_input", "lmoe_moe_tail",
                            "lmoe_block_forward"]), names


def test_library_exports_every_declared_symbol(lm):
    lib = ctypes.CDLL(lm.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(lm.EXPORTS) == set(_declared())


def test_stage_names(lm):
    assert [lm.stage_name(i) for i in range(lm.NUM_STAGE_EVENTS)] == list(lm.STAGES)
    assert lm.stage_name(-1) == "?" and lm.stage_name(lm.NUM_STAGE_EVENTS) == "?"


def test_traced_forward_rejects_missing_events(lm):
    d = lm._dims(K3)
    w = _weights(lm)
    ev = (ctypes.c_void_p * lm.NUM_STAGE_EVENTS)(*([0x1000] * (lm.NUM_STAGE_EVENTS - 1) + [0]))
    f = lm._lib.lmoe_forward_traced
    assert f(ctypes.byref(d), 0x20000000, ctypes.byref(w), 0, None, 0x30000000, 0x40000000, 1,
             None, None) == lm.LMOE_ERR_NULL
    assert f(ctypes.byref(d), 0x20000000, ctypes.byref(w), 0, None, 0x30000000, 0x40000000, 1,
             None, ev) == lm.LMOE_ERR_NULL


def test_path_names(lm):
    assert lm.path_name(K3) == "fused_decode"
    assert lm.path_name(K3, True) == "fused_decode"   # given logits are published
    # two and three K3 tokens: one kernel, one token per MFMA row; from four
    # the grouped kernels stream the weights faster
    for T in (2, 3):
        assert lm.path_name((T,) + K3[1:]) == "fused_multi"
        assert lm.path_name((T,) + K3[1:], True) == "fused_multi"
    for T in (4, 5, 16, 17):
        assert lm.path_name((T,) + K3[1:]) == "grouped"
    assert lm.path_name((64,) + K3[1:]) == "grouped"
    assert lm.path_name((4096,) + K3[1:]) == "grouped"
    assert lm.path_name((1, 8192, 896, 16, 2048, 2, 2048)) == "grouped"  # L too wide
    # per-expert widths up to 4096 decode in one kernel, whatever S * Is
    assert lm.path_name((1, 3584, 896, 16, 3072, 2, 3072)) == "fused_decode"
    assert lm.path_name((1, 3584, 896, 16, 256, 8, 4096)) == "fused_decode"
    assert lm.path_name((1, 3584, 896, 16, 2048, 2, 4128)) == "grouped"
    assert lm.path_name((1, 3583, 896, 16, 2048, 2, 2048)) == "invalid"


def test_status_strings(lm):
    for code in range(6):
        assert lm.status_string(code)
    assert lm.status_string(0) == "ok"
    assert "unknown" in lm.status_string(99)


K3 = (1, 3584, 896, 16, 2048, 2, 2048)


def test_workspace_bytes_valid_and_invalid(lm):
    assert lm.workspace_bytes(K3) > 0
    big = lm.workspace_bytes((4096,) + K3[1:])
    assert big > lm.workspace_bytes(K3)
    # T=8192: route partials dominate (131072 routes x 3584 fp32)
    w8 = lm.workspace_bytes((8192,) + K3[1:])
    assert w8 >= 131072 * 3584 * 4
    for bad in [(1, 3583, 896, 16, 2048, 2, 2048),   # L % 32
                (1, 3584, 1025, 16, 2048, 2, 2048),  # E > 1024
                (1, 3584, 896, 33, 2048, 2, 2048),   # k > 32
                (1, 3584, 8, 9, 2048, 2, 2048),      # k > E
                (1, 3584, 896, 16, 2040, 2, 2048),   # I % 32
                (1, 3584, 896, 16, 2048, 2, 100),    # Is % 32
                (-1, 3584, 896, 16, 2048, 2, 2048),
                (1, 3584, 896, 0, 2048, 2, 2048)]:
        assert lm.workspace_bytes(bad) == 0, bad
    assert lm.workspace_bytes((0,) + K3[1:]) > 0


def _weights(lm, base=0x10000000):
    vals = [base + 0x100000 * i for i in range(10)]
    return lm.lmoe_weights(*vals)


def _call_forward(lm, dims, x=0x20000000, w=None, logits_given=0, r=None, out=0x30000000,
                  ws=0x40000000, ws_bytes=None):
    d = lm._dims(dims)
    if w is None:
        w = _weights(lm)
    if ws_bytes is None:
        ws_bytes = 1
    return lm._lib.lmoe_forward(ctypes.byref(d), x, ctypes.byref(w), logits_given,
                                ctypes.byref(r) if r is not None else None, out, ws,
                                ws_bytes, None)


def test_forward_rejects_bad_arguments(lm):
    assert lm._lib.lmoe_forward(None, 0, None, 0, None, 0, 0, 0, None) == lm.LMOE_ERR_NULL
    assert _call_forward(lm, (1, 3583, 896, 16, 2048, 2, 2048)) == lm.LMOE_ERR_SHAPE
    assert _call_forward(lm, K3, x=None) == lm.LMOE_ERR_NULL
    assert _call_forward(lm, K3, out=None) == lm.LMOE_ERR_NULL
    assert _call_forward(lm, K3, ws=None) == lm.LMOE_ERR_NULL
    w = _weights(lm)
    w.gate_s = None
    assert _call_forward(lm, K3, w=w) == lm.LMOE_ERR_NULL
    w = _weights(lm)
    w.sh_down = None
    assert _call_forward(lm, K3, w=w) == lm.LMOE_ERR_NULL
    # logits given without a routing struct / without logits
    assert _call_forward(lm, K3, logits_given=1) == lm.LMOE_ERR_NULL
    assert _call_forward(lm, K3, logits_given=1, r=lm.lmoe_routing()) == lm.LMOE_ERR_NULL
    # misaligned pointers
    assert _call_forward(lm, K3, x=0x20000008) == lm.LMOE_ERR_ALIGN
    w = _weights(lm)
    w.down_q = 0x10000001
    assert _call_forward(lm, K3, w=w) == lm.LMOE_ERR_ALIGN
    r = lm.lmoe_routing()
    r.perm = 0x50000004
    assert _call_forward(lm, K3, r=r) == lm.LMOE_ERR_ALIGN
    # workspace one byte short
    need = lm.workspace_bytes(K3)
    assert _call_forward(lm, K3, ws_bytes=need - 1) == lm.LMOE_ERR_WORKSPACE


def test_forward_zero_tokens_needs_no_pointers(lm):
    d = lm._dims((0,) + K3[1:])
    w = lm.lmoe_weights()
    assert lm._lib.lmoe_forward(ctypes.byref(d), None, ctypes.byref(w), 0, None, None, None,
                                0, None) == lm.LMOE_OK


def test_route_rejects_bad_arguments(lm):
    d = lm._dims(K3)
    assert lm._lib.lmoe_route(ctypes.byref(d), None, None, 0, None, 0x40000000, 1 << 40,
                              None) == lm.LMOE_ERR_NULL
    assert lm._lib.lmoe_route(ctypes.byref(d), 0x20000000, 0x21000000, 0, None, None, 0,
                              None) == lm.LMOE_ERR_NULL
    assert lm._lib.lmoe_route(ctypes.byref(d), 0x20000000, 0x21000000, 0, None, 0x40000000,
                              16, None) == lm.LMOE_ERR_WORKSPACE
    bad = lm._dims((1, 3584, 896, 17, 2048, 2, 2048 + 1))
    assert lm._lib.lmoe_route(ctypes.byref(bad), 0x20000000, 0x21000000, 0, None,
                              0x40000000, 1 << 40, None) == lm.LMOE_ERR_SHAPE


def test_dequant_hook_rejects_bad_arguments(lm):
    f = lm._lib.lmoe_debug_dequant_mxfp4
    assert f(0x1000, 0x2000, 4, 48, 0x3000, None) == lm.LMOE_ERR_SHAPE
    assert f(0x1000, 0x2000, -1, 64, 0x3000, None) == lm.LMOE_ERR_SHAPE
    assert f(None, 0x2000, 4, 64, 0x3000, None) == lm.LMOE_ERR_NULL
    assert f(0x1008, 0x2000, 4, 64, 0x3000, None) == lm.LMOE_ERR_ALIGN
    assert f(0x1000, 0x2000, 0, 64, 0x3000, None) == lm.LMOE_OK


def test_quantize_hook_rejects_bad_arguments(lm):
    f = lm._lib.lmoe_debug_quantize_act
    assert f(0x1000, 4, 48, lm.ACT_E4M3, 0x2000, 0x3000, None) == lm.LMOE_ERR_SHAPE
    assert f(0x1000, -1, 64, lm.ACT_E4M3, 0x2000, 0x3000, None) == lm.LMOE_ERR_SHAPE
    assert f(0x1000, 4, 64, lm.ACT_BF16, 0x2000, 0x3000, None) == lm.LMOE_ERR_SHAPE
    assert f(0x1000, 4, 64, 7, 0x2000, 0x3000, None) == lm.LMOE_ERR_SHAPE
    assert f(None, 4, 64, lm.ACT_E2M1, 0x2000, 0x3000, None) == lm.LMOE_ERR_NULL
    assert f(0x1000, 4, 64, lm.ACT_E2M1, 0x2000, None, None) == lm.LMOE_ERR_NULL
    assert f(0x1008, 4, 64, lm.ACT_E2M1, 0x2000, 0x3000, None) == lm.LMOE_ERR_ALIGN
    assert f(0x1000, 0, 64, lm.ACT_E2M1, 0x2000, 0x3000, None) == lm.LMOE_OK


def test_act_format_rejected_outside_the_packed_path(lm):
    """Quantised activations run only on tile-packed experts with L and I
    multiples of 128; every other request is refused on the host."""
    d = lm._dims(K3)
    w = _weights(lm)
    for act in (lm.ACT_E4M3, lm.ACT_E2M1, 3):
        ex = lm.lmoe_exec(None, None, None, None, 0, act)
        assert lm._lib.lmoe_forward_ex(ctypes.byref(d), 0x20000000, ctypes.byref(w), 0, None,
                                       0x30000000, 0x40000000, 1 << 40, None,
                                       ctypes.byref(ex)) == lm.LMOE_ERR_SHAPE
    P = (0x50000000, 0x51000000, 0x52000000, 0x53000000)
    pw = lm.lmoe_packed_weights(0x10000000, *P, 0x11000000, 0x12000000, 0x13000000)
    odd = lm._dims((4, 3584 - 32, 896, 16, 2048, 2, 2048))     # L % 128 != 0
    ex = lm.lmoe_exec(None, None, None, None, 0, lm.ACT_E2M1)
    assert lm._lib.lmoe_forward_packed(ctypes.byref(odd), 0x20000000, ctypes.byref(pw), 0, None,
                                       0x30000000, 0x40000000, 1 << 40, None,
                                       ctypes.byref(ex)) == lm.LMOE_ERR_SHAPE
    bad = lm.lmoe_exec(None, None, None, None, 0, 5)
    assert lm._lib.lmoe_forward_packed(ctypes.byref(d), 0x20000000, ctypes.byref(pw), 0, None,
                                       0x30000000, 0x40000000, 1 << 40, None,
                                       ctypes.byref(bad)) == lm.LMOE_ERR_SHAPE


def test_forward_ex_rejects_bad_arguments(lm):
    d = lm._dims(K3)
    w = _weights(lm)
    f = lm._lib.lmoe_forward_ex
    # a side stream without its fork or join event; a missing stage event
    ev = (ctypes.c_void_p * lm.NUM_STAGE_EVENTS)(*([0x1000] * (lm.NUM_STAGE_EVENTS - 1) + [0]))
    traced = lm.lmoe_exec(None, None, None, ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)))
    for ex in (lm.lmoe_exec(0x1000, None, 0x3000), lm.lmoe_exec(0x1000, 0x2000, None), traced):
        assert f(ctypes.byref(d), 0x20000000, ctypes.byref(w), 0, None, 0x30000000, 0x40000000,
                 1 << 40, None, ctypes.byref(ex)) == lm.LMOE_ERR_NULL
        d0 = lm._dims((0,) + K3[1:])
        assert f(ctypes.byref(d0), None, ctypes.byref(w), 0, None, None, None, 0, None,
                 ctypes.byref(ex)) == lm.LMOE_ERR_NULL
    # an unknown path choice
    odd = lm.lmoe_exec(None, None, None, None, 7)
    assert f(ctypes.byref(d), 0x20000000, ctypes.byref(w), 0, None, 0x30000000, 0x40000000,
             1 << 40, None, ctypes.byref(odd)) == lm.LMOE_ERR_SHAPE
    # the same argument checks as lmoe_forward
    assert f(None, 0, None, 0, None, 0, 0, 0, None, None) == lm.LMOE_ERR_NULL
    bad = lm._dims((1, 3583, 896, 16, 2048, 2, 2048))
    assert f(ctypes.byref(bad), 0x20000000, ctypes.byref(w), 0, None, 0x30000000, 0x40000000,
             1 << 40, None, None) == lm.LMOE_ERR_SHAPE
    assert f(ctypes.byref(d), 0x20000008, ctypes.byref(w), 0, None, 0x30000000, 0x40000000,
             1 << 40, None, None) == lm.LMOE_ERR_ALIGN
    assert f(ctypes.byref(d), 0x20000000, ctypes.byref(w), 0, None, 0x30000000, 0x40000000,
             lm.workspace_bytes(K3) - 1, None, None) == lm.LMOE_ERR_WORKSPACE
    d0 = lm._dims((0,) + K3[1:])
    assert f(ctypes.byref(d0), None, ctypes.byref(lm.lmoe_weights()), 0, None, None, None, 0,
             None, None) == lm.LMOE_OK


def test_forward_noalloc_rejects_on_the_host(lm):
    """Rejections that return before the device is touched."""
    f = lm._lib.lmoe_forward_noalloc
    w = _weights(lm)
    assert f(None, 0x20000000, ctypes.byref(w), 0, None, 0x30000000, None) == lm.LMOE_ERR_NULL
    bad = lm._dims((1, 3583, 896, 16, 2048, 2, 2048))
    assert f(ctypes.byref(bad), 0x20000000, ctypes.byref(w), 0, None, 0x30000000,
             None) == lm.LMOE_ERR_SHAPE
    # the scratch holds the workspace of up to about 150 Kimi-K3 tokens
    for T in (1, 64, 128):
        assert lm.workspace_bytes((T,) + K3[1:]) <= lm.NOALLOC_SCRATCH_BYTES, T
    big = (4096,) + K3[1:]
    assert lm.workspace_bytes(big) > lm.NOALLOC_SCRATCH_BYTES
    d = lm._dims(big)
    assert f(ctypes.byref(d), 0x20000000, ctypes.byref(w), 0, None, 0x30000000,
             None) == lm.LMOE_ERR_WORKSPACE
    d0 = lm._dims((0,) + K3[1:])
    assert f(ctypes.byref(d0), None, ctypes.byref(lm.lmoe_weights()), 0, None, None,
             None) == lm.LMOE_OK


def test_header_scratch_size_matches_binding(lm):
    text = open(HEADER).read()
    m = re.search(r"#define LMOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == lm.NOALLOC_SCRATCH_BYTES


def test_packed_sizes(lm):
    z = lm.packed_sizes(K3)
    # Kimi-K3 widths need no padding: the packed arrays hold exactly the
    # row-major bytes
    assert z["gu_q"] == 896 * 2 * 2048 * 3584 // 2
    assert z["down_q"] == 896 * 3584 * 2048 // 2
    assert z["gu_s"] == 896 * 2 * 2048 * 3584 // 32
    assert z["down_s"] == 896 * 3584 * 2048 // 32
    # ragged widths pad rows to 32 and K to 128 (codes) / 512 (exponents)
    z = lm.packed_sizes((1, 416, 48, 6, 352, 2, 224))
    assert z["gu_q"] == 48 * (704 // 32) * 4 * 2048
    assert z["down_q"] == 48 * 13 * 3 * 2048
    with pytest.raises(lm.LmoeError):
        lm.packed_sizes((1, 3583, 896, 16, 2048, 2, 2048))


def test_pack_and_forward_packed_reject_bad_arguments(lm):
    d = lm._dims(K3)
    w = _weights(lm)
    f = lm._lib.lmoe_pack_weights
    P = (0x50000000, 0x51000000, 0x52000000, 0x53000000)
    assert f(None, ctypes.byref(w), *P, None) == lm.LMOE_ERR_NULL
    assert f(ctypes.byref(d), ctypes.byref(w), None, *P[1:], None) == lm.LMOE_ERR_NULL
    assert f(ctypes.byref(d), ctypes.byref(w), P[0] + 8, *P[1:], None) == lm.LMOE_ERR_ALIGN
    bad = lm._dims((1, 3583, 896, 16, 2048, 2, 2048))
    assert f(ctypes.byref(bad), ctypes.byref(w), *P, None) == lm.LMOE_ERR_SHAPE
    g = lm._lib.lmoe_forward_packed
    pw = lm.lmoe_packed_weights(0x10000000, *P, 0x11000000, 0x12000000, 0x13000000)
    assert g(ctypes.byref(d), 0x20000000, None, 0, None, 0x30000000, 0x40000000, 1 << 40,
             None, None) == lm.LMOE_ERR_NULL
    pw0 = lm.lmoe_packed_weights(0x10000000, None, *P[1:], 0x11000000, 0x12000000, 0x13000000)
    assert g(ctypes.byref(d), 0x20000000, ctypes.byref(pw0), 0, None, 0x30000000, 0x40000000,
             1 << 40, None, None) == lm.LMOE_ERR_NULL
    pw1 = lm.lmoe_packed_weights(0x10000000, P[0] + 4, *P[1:], 0x11000000, 0x12000000,
                                 0x13000000)
    assert g(ctypes.byref(d), 0x20000000, ctypes.byref(pw1), 0, None, 0x30000000, 0x40000000,
             1 << 40, None, None) == lm.LMOE_ERR_ALIGN
    assert g(ctypes.byref(d), 0x20000000, ctypes.byref(pw), 0, None, 0x30000000, 0x40000000,
             lm.workspace_bytes(K3) - 1, None, None) == lm.LMOE_ERR_WORKSPACE
    d0 = lm._dims((0,) + K3[1:])
    assert g(ctypes.byref(d0), None, ctypes.byref(pw), 0, None, None, None, 0, None,
             None) == lm.LMOE_OK


def test_wait_errors_rejects_bad_arguments(lm):
    f = lm._lib.lmoe_wait_errors
    assert f(None, 1 << 20, 0x2000, None) == lm.LMOE_ERR_NULL
    assert f(0x40000000, 1 << 20, None, None) == lm.LMOE_ERR_NULL
    assert f(0x40000008, 1 << 20, 0x2000, None) == lm.LMOE_ERR_ALIGN
    assert f(0x40000000, 1 << 20, 0x2002, None) == lm.LMOE_ERR_ALIGN
    assert f(0x40000000, 32767, 0x2000, None) == lm.LMOE_ERR_WORKSPACE


def test_read_stream_rejects_bad_arguments(lm):
    f = lm._lib.lmoe_debug_read_stream
    assert f(None, 1024, 0x2000, 4, None) == lm.LMOE_ERR_NULL
    assert f(0x1000, 1024, None, 4, None) == lm.LMOE_ERR_NULL
    assert f(0x1000, 1000, 0x2000, 4, None) == lm.LMOE_ERR_SHAPE
    assert f(0x1000, 1024, 0x2000, 0, None) == lm.LMOE_ERR_SHAPE
    assert f(0x1000, 1024, 0x2000, 65537, None) == lm.LMOE_ERR_SHAPE
    assert f(0x1008, 1024, 0x2000, 4, None) == lm.LMOE_ERR_ALIGN
    assert f(0x1000, 1024, 0x2002, 4, None) == lm.LMOE_ERR_ALIGN
    assert f(0x1000, 0, 0x2000, 4, None) == lm.LMOE_OK


def test_mfma_rate_rejects_bad_arguments(lm):
    f = lm._lib.lmoe_debug_mfma_rate
    assert f(16, None, 4, None) == lm.LMOE_ERR_NULL
    assert f(-1, 0x2000, 4, None) == lm.LMOE_ERR_SHAPE
    assert f(16, 0x2000, 0, None) == lm.LMOE_ERR_SHAPE
    assert f(16, 0x2000, 65537, None) == lm.LMOE_ERR_SHAPE
    assert f(16, 0x2002, 4, None) == lm.LMOE_ERR_ALIGN


def test_binding_rejects_host_tensors(lm):
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        lm._ptr(torch.zeros(4))


K3_BLOCK = (1, 7168, 3584, 896, 16, 2048, 2, 2048)   # T, H, L, E, k, I, S, Is


def test_block_workspace_bytes_valid_and_invalid(lm):
    assert lm.block_workspace_bytes(K3_BLOCK) > lm.workspace_bytes(
        (1, 3584, 896, 16, 2048, 0, 0))
    assert lm.block_workspace_bytes((4096,) + K3_BLOCK[1:]) > lm.block_workspace_bytes(K3_BLOCK)
    assert lm.block_workspace_bytes((1, 7168, 3584, 896, 16, 2048, 0, 0)) > 0
    for bad in [(1, 7160, 3584, 896, 16, 2048, 2, 2048),   # H % 64
                (1, 7168, 3552, 896, 16, 2048, 2, 2048),   # L % 64
                (1, 7168, 3584, 900, 16, 2048, 2, 2048),   # E % 32
                (1, 7168, 3584, 896, 16, 2048, 1, 32),     # S * Is % 64
                (1, 7168, 3584, 896, 16, 2048, 9, 2048),   # S > 8
                (1, 7168, 3584, 896, 33, 2048, 2, 2048),   # k > 32
                (-1, 7168, 3584, 896, 16, 2048, 2, 2048)]:
        assert lm.block_workspace_bytes(bad) == 0, bad


def test_block_calls_reject_bad_arguments_on_the_host(lm):
    d = lm.lmoe_block_dims(*K3_BLOCK)
    big = 1 << 40
    p = [0x10000000 + 0x100000 * i for i in range(12)]
    mi, mt = lm._lib.lmoe_moe_input, lm._lib.lmoe_moe_tail
    assert mi(None, p[0], p[1], p[2], p[3], p[4], p[5], big, None) == lm.LMOE_ERR_NULL
    assert mi(ctypes.byref(d), None, p[1], p[2], p[3], p[4], p[5], big, None) == lm.LMOE_ERR_NULL
    assert mi(ctypes.byref(d), p[0], p[1], p[2], p[3], None, p[5], big, None) == lm.LMOE_ERR_NULL
    assert mi(ctypes.byref(d), p[0] + 8, p[1], p[2], p[3], p[4], p[5], big,
              None) == lm.LMOE_ERR_ALIGN
    assert mi(ctypes.byref(d), p[0], p[1], p[2], p[3], p[4], p[5], 1024,
              None) == lm.LMOE_ERR_WORKSPACE
    bad = lm.lmoe_block_dims(1, 7160, 3584, 896, 16, 2048, 2, 2048)
    assert mi(ctypes.byref(bad), p[0], p[1], p[2], p[3], p[4], p[5], big,
              None) == lm.LMOE_ERR_SHAPE
    assert mt(ctypes.byref(d), p[0], p[1], p[2], p[3], None, p[5], p[6], p[7], big,
              None) == lm.LMOE_ERR_NULL
    assert mt(ctypes.byref(d), p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], 1024,
              None) == lm.LMOE_ERR_WORKSPACE
    bw = lm.lmoe_block_weights(p[0], p[1], p[2], None)
    w = lm.lmoe_weights(*[p[3]] * 10)
    bf = lm._lib.lmoe_block_forward
    assert bf(ctypes.byref(d), p[4], p[5], ctypes.byref(bw), ctypes.byref(w), None, p[6], p[7],
              big, None) == lm.LMOE_ERR_NULL          # S > 0 needs w_sd
    assert bf(ctypes.byref(d), p[4], p[5], None, ctypes.byref(w), None, p[6], p[7], big,
              None) == lm.LMOE_ERR_NULL
    d0 = lm.lmoe_block_dims(0, *K3_BLOCK[1:])
    assert bf(ctypes.byref(d0), None, None, ctypes.byref(bw), ctypes.byref(w), None, None, None,
              0, None) == lm.LMOE_OK


def test_packed_forward_rejects_offsets_beyond_32_bits(lm):
    """The packed GEMMs address activation rows with 32-bit byte offsets:
    T * k * I (and T * L) must stay below 2^31."""
    pw = lm.lmoe_packed_weights(*[0x10000000 + 0x100000 * i for i in range(8)])
    for T, want in ((65536, lm.LMOE_ERR_SHAPE), (65535, lm.LMOE_ERR_WORKSPACE)):
        d = lm.lmoe_dims(T, 3584, 896, 16, 2048, 2, 2048)
        assert lm._lib.lmoe_forward_packed(ctypes.byref(d), 0x20000000, ctypes.byref(pw), 0, None,
                                           0x30000000, 0x40000000, 1024, None, None) == want, T

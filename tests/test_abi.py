"""The C ABI library: it builds for gfx950, loads, exports every function the
header declares, and rejects invalid arguments with the documented status
before touching the GPU.  CPU only: no call here launches a kernel."""
import ctypes
import os
import subprocess

import pytest

import w8a8_int8_quantized_bf16_amd as w8

OK, INVALID, SHAPE, ALIGN, WS_SMALL, HIP, SCRATCH = 0, -1, -2, -3, -4, -5, -6
FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced: every call below returns before any launch
MIS = ctypes.c_void_p((1 << 20) + 4)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(w8.LIB_PATH):
        from w8a8_int8_quantized_bf16_amd import build
        build.build()
    return w8.lib()


def test_exports_every_declared_function(L):
    names = w8.header_functions()
    assert len(names) == 26
    for n in ("w8a8_quant_act", "moe_route_topk", "moe_permute", "w8a8_grouped_gemm", "moe_combine",
              "w8a8_moe_layer", "w4a8_quant_weights", "w4a8_pack_weights", "w4a8_grouped_gemm", "w8a8_linear",
              "w8a8_linear_q", "w8a8_linear_workspace_size", "w8a8_linear_q_workspace_size",
              "w8a8_grouped_gemm_noalloc"):
        assert n in names
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", w8.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported


def test_library_holds_gfx950_code(L):
    """The device code objects embedded in the library target gfx950 only."""
    blob = open(w8.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob
    assert b"amdgcn-amd-amdhsa--gfx942" not in blob


def test_status_strings(L):
    for code in (OK, INVALID, SHAPE, ALIGN, WS_SMALL, HIP, SCRATCH):
        assert w8.status_string(code)
    assert w8.status_string(-99) == "unknown status"


def test_quant_act_rejects(L):
    s = None
    assert L.w8a8_quant_act(FAKE, 0, 4, 24, 24, FAKE, FAKE, s) == SHAPE       # cols % 16
    assert L.w8a8_quant_act(FAKE, 0, 4, 32, 16, FAKE, FAKE, s) == INVALID     # ld < cols
    assert L.w8a8_quant_act(FAKE, 7, 4, 32, 32, FAKE, FAKE, s) == INVALID     # dtype
    assert L.w8a8_quant_act(None, 0, 4, 32, 32, FAKE, FAKE, s) == INVALID
    assert L.w8a8_quant_act(MIS, 0, 4, 32, 32, FAKE, FAKE, s) == ALIGN
    assert L.w8a8_quant_act(FAKE, 0, 4, 32, 36, FAKE, FAKE, s) == ALIGN       # 72-byte rows
    assert L.w8a8_quant_act(FAKE, 0, -1, 32, 32, FAKE, FAKE, s) == INVALID
    assert L.w8a8_quant_act(None, 0, 0, 32, 32, None, None, s) == OK          # empty: no-op


def test_route_rejects(L):
    s = None
    assert L.moe_route_topk(FAKE, 0, FAKE, 8, 64, 8, 9, 1, FAKE, FAKE, None, s) == INVALID   # k > E
    assert L.moe_route_topk(FAKE, 0, FAKE, 8, 64, 300, 8, 1, FAKE, FAKE, None, s) == SHAPE  # E > 256
    assert L.moe_route_topk(FAKE, 0, FAKE, 8, 72, 8, 2, 1, FAKE, FAKE, None, s) == SHAPE    # H % 16
    assert L.moe_route_topk(FAKE, 0, None, 8, 64, 8, 2, 1, FAKE, FAKE, None, s) == INVALID
    assert L.moe_route_topk(FAKE, 0, FAKE, 8, 64, 8, 2, 1, MIS, FAKE, None, s) == ALIGN
    assert L.moe_route_topk(FAKE, 2, FAKE, 8, 64, 8, 2, 1, FAKE, FAKE, None, s) == INVALID  # dtype
    assert L.moe_route_topk(None, 0, None, 0, 64, 8, 2, 1, None, None, None, s) == OK
    # the variant with the packed copy: the same checks, and that copy's alignment
    assert L.moe_route_topk_packed(FAKE, 0, FAKE, FAKE, 8, 72, 8, 2, 1, FAKE, FAKE, None, s) == SHAPE
    assert L.moe_route_topk_packed(FAKE, 0, FAKE, FAKE, 8, 64, 8, 9, 1, FAKE, FAKE, None, s) == INVALID
    assert L.moe_route_topk_packed(FAKE, 0, FAKE, MIS, 8, 64, 8, 2, 1, FAKE, FAKE, None, s) == ALIGN
    assert L.moe_route_topk_packed(None, 0, None, None, 0, 64, 8, 2, 1, None, None, None, s) == OK


def test_permute_rejects(L):
    s = None
    need = L.moe_permute_workspace_size(4096, 8, 128)
    assert need >= 16 * 128 * 4
    assert L.moe_permute(FAKE, 4096, 8, 128, FAKE, FAKE, FAKE, FAKE, need - 1, s) == WS_SMALL
    assert L.moe_permute(FAKE, 4096, 8, 4, FAKE, FAKE, FAKE, FAKE, need, s) == INVALID       # k > E
    assert L.moe_permute(FAKE, 16, 2, 512, FAKE, FAKE, FAKE, FAKE, need, s) == SHAPE
    assert L.moe_permute(FAKE, 16, 2, 8, FAKE, MIS, FAKE, FAKE, need, s) == ALIGN
    assert L.moe_permute(FAKE, 16, 2, 8, None, FAKE, FAKE, FAKE, need, s) == INVALID


def test_grouped_gemm_rejects(L):
    s = None
    ws = L.w8a8_grouped_gemm_workspace_size(1024, 256, 8)
    args = lambda **kw: [kw.get("A", FAKE), kw.get("Arows", 1024), kw.get("sa", FAKE), kw.get("gat", None),
                         kw.get("div", 1),
                         kw.get("B", FAKE), kw.get("lay", 0), kw.get("sb", FAKE), kw.get("off", FAKE), kw.get("G", 8),
                         kw.get("M", 1024), kw.get("N", 256), kw.get("K", 256), kw.get("epi", 1),
                         kw.get("od", 0), kw.get("out", FAKE), kw.get("ws", FAKE), kw.get("wsb", ws), s]
    assert L.w8a8_grouped_gemm(*args(K=200)) == SHAPE
    assert L.w8a8_grouped_gemm(*args(N=200)) == SHAPE
    assert L.w8a8_grouped_gemm(*args(N=288, epi=2)) == SHAPE                  # SwiGLU needs N % 64
    assert L.w8a8_grouped_gemm(*args(lay=2)) == INVALID
    assert L.w8a8_grouped_gemm(*args(epi=3)) == INVALID
    assert L.w8a8_grouped_gemm(*args(epi=0, od=0)) == INVALID                 # RAW needs int32 out
    assert L.w8a8_grouped_gemm(*args(od=2)) == INVALID                        # dequant cannot be int32
    assert L.w8a8_grouped_gemm(*args(sb=None)) == INVALID
    assert L.w8a8_grouped_gemm(*args(gat=FAKE, div=0)) == INVALID
    assert L.w8a8_grouped_gemm(*args(A=MIS)) == ALIGN
    assert L.w8a8_grouped_gemm(*args(wsb=ws - 1)) == WS_SMALL
    assert L.w8a8_grouped_gemm(*args(G=0)) == INVALID
    assert L.w8a8_grouped_gemm(*args(M=0, A=None, out=None)) == OK
    assert L.w8a8_grouped_gemm(*args(Arows=1 << 20, K=4096)) == SHAPE        # 32-bit offsets
    assert L.w8a8_grouped_gemm(*args(Arows=-1)) == INVALID


def test_grouped_gemm_noalloc_rejects(L):
    """The allocation-free grouped GEMM checks the arguments of
    w8a8_grouped_gemm and refuses, before any launch, a problem whose tile
    table exceeds its fixed scratch array."""
    s = None
    args = lambda **kw: [kw.get("A", FAKE), kw.get("Arows", 1024), kw.get("sa", FAKE), kw.get("gat", None),
                         kw.get("div", 1), kw.get("B", FAKE), kw.get("lay", 0), kw.get("sb", FAKE),
                         kw.get("off", FAKE), kw.get("G", 8), kw.get("M", 1024), kw.get("N", 256), kw.get("K", 256),
                         kw.get("epi", 1), kw.get("od", 0), kw.get("out", FAKE), s]
    assert L.w8a8_grouped_gemm_noalloc(*args(K=200)) == SHAPE
    assert L.w8a8_grouped_gemm_noalloc(*args(epi=0, od=0)) == INVALID
    assert L.w8a8_grouped_gemm_noalloc(*args(A=MIS)) == ALIGN
    assert L.w8a8_grouped_gemm_noalloc(*args(off=None)) == INVALID
    assert L.w8a8_grouped_gemm_noalloc(*args(M=0, A=None, out=None)) == OK
    limit = 4 << 20
    # the tile table of the 235B layer's GEMMs (65,536 rows and a shared group) fits; 4M rows do not
    assert L.w8a8_grouped_gemm_workspace_size(65536, 4096, 129) <= limit
    big = 1 << 22
    assert L.w8a8_grouped_gemm_workspace_size(big, 4096, 1) > limit
    assert L.w8a8_grouped_gemm_noalloc(*args(M=big, G=1, N=4096, gat=FAKE, div=8)) == SCRATCH
    assert w8.status_string(SCRATCH) != "unknown status"


def test_pack_rejects(L):
    s = None
    assert L.w8a8_packed_weights_size(2, 100, 200) == 2 * 4 * 2 * 4096
    assert L.w8a8_pack_weights(FAKE, 2, 40, 64, FAKE, s) == SHAPE
    assert L.w8a8_pack_weights(FAKE, 0, 48, 64, FAKE, s) == INVALID
    assert L.w8a8_pack_weights(MIS, 1, 48, 64, FAKE, s) == ALIGN
    assert L.w8a8_pack_weights(None, 1, 48, 64, FAKE, s) == INVALID


def test_router_widen_rejects(L):
    s = None
    assert L.moe_router_widen(FAKE, 8, 72, FAKE, s) == SHAPE
    assert L.moe_router_widen(FAKE, 0, 64, FAKE, s) == INVALID
    assert L.moe_router_widen(None, 8, 64, FAKE, s) == INVALID
    assert L.moe_router_widen(FAKE, 8, 64, MIS, s) == ALIGN


def test_router_pack_rejects(L):
    s = None
    assert L.moe_router_pack(FAKE, 8, 72, FAKE, s) == SHAPE
    assert L.moe_router_pack(FAKE, 0, 64, FAKE, s) == INVALID
    assert L.moe_router_pack(FAKE, 8, 64, None, s) == INVALID
    assert L.moe_router_pack(MIS, 8, 64, FAKE, s) == ALIGN
    assert L.moe_router_pack(FAKE, 8, 64, MIS, s) == ALIGN


def test_combine_rejects(L):
    s = None
    assert L.moe_combine(FAKE, 0, FAKE, FAKE, 16, 2, 72, FAKE, 0, s) == SHAPE
    assert L.moe_combine(FAKE, 3, FAKE, FAKE, 16, 2, 64, FAKE, 0, s) == INVALID
    assert L.moe_combine(FAKE, 0, FAKE, None, 16, 2, 64, FAKE, 0, s) == INVALID
    assert L.moe_combine(FAKE, 0, FAKE, FAKE, 16, 2, 64, MIS, 0, s) == ALIGN
    assert L.moe_combine(None, 0, None, None, 0, 2, 64, None, 0, s) == OK


def _weights(E=8, k=2, H=64, I=32, ptr=FAKE):
    return w8._Weights(E, k, H, I, ptr.value, ptr.value, ptr.value, ptr.value, ptr.value, None, None,
                       0, None, None, None, None, None)


def _with_shared(W, Is=64, ptr=FAKE):
    W.I_shared = Is
    W.w_shared_gate_up = W.s_shared_gate_up = W.w_shared_down = W.s_shared_down = W.w_shared_gate = ptr.value
    return W


def test_layer_rejects_and_sizes_workspace(L):
    s = None
    W = _weights()
    need = L.w8a8_moe_layer_workspace_size(ctypes.byref(W), 16, 1)
    # ids, w, xq, sx, offsets, sorted, pos, h, hq, sh, y (int16) + exponents, permute, gemm map
    assert need >= 32 * 4 * 4 + 16 * 64 + 32 * 32 * 3 + 32 * 64 * 2 + 32
    assert L.w8a8_moe_layer(ctypes.byref(W), FAKE, 1, 16, FAKE, FAKE, need - 1, s) == WS_SMALL
    assert L.w8a8_moe_layer(ctypes.byref(W), FAKE, 1, 16, FAKE, MIS, need, s) == ALIGN
    assert L.w8a8_moe_layer(ctypes.byref(W), FAKE, 5, 16, FAKE, FAKE, need, s) == INVALID
    assert L.w8a8_moe_layer(ctypes.byref(_weights(H=72)), FAKE, 1, 16, FAKE, FAKE, need, s) == SHAPE
    assert L.w8a8_moe_layer(ctypes.byref(_weights(I=48)), FAKE, 1, 16, FAKE, FAKE, need, s) == SHAPE
    assert L.w8a8_moe_layer(ctypes.byref(_weights(k=9)), FAKE, 1, 16, FAKE, FAKE, need, s) == INVALID
    assert L.w8a8_moe_layer(ctypes.byref(_weights(E=257, k=2)), FAKE, 1, 16, FAKE, FAKE, need, s) == SHAPE
    assert L.w8a8_moe_layer(ctypes.byref(_weights(ptr=MIS)), FAKE, 1, 16, FAKE, FAKE, need, s) == ALIGN
    Wf = _weights()
    Wf.w_gate_f32 = MIS.value
    assert L.w8a8_moe_layer(ctypes.byref(Wf), FAKE, 1, 16, FAKE, FAKE, need, s) == ALIGN
    assert L.w8a8_moe_layer(None, FAKE, 1, 16, FAKE, FAKE, need, s) == INVALID
    assert L.w8a8_moe_layer(ctypes.byref(W), None, 1, 0, None, None, 0, s) == OK
    # W4A8 gate_up: the packed W4 buffer (codes, scales, offsets) replaces the int8 gate_up
    W4 = _weights()
    W4.w4_gate_up, W4.w_gate_up, W4.s_gate_up = MIS.value, None, None
    assert L.w8a8_moe_layer(ctypes.byref(W4), FAKE, 1, 16, FAKE, FAKE, need, s) == ALIGN
    W4.w4_gate_up = FAKE.value
    assert L.w8a8_moe_layer(ctypes.byref(W4), FAKE, 1, 16, FAKE, FAKE, need - 1, s) == WS_SMALL
    W4.w4_gate_up = None
    assert L.w8a8_moe_layer(ctypes.byref(W4), FAKE, 1, 16, FAKE, FAKE, need, s) == INVALID
    # shared expert: all of its weights or none, I_shared a multiple of 32
    needs = L.w8a8_moe_layer_workspace_size(ctypes.byref(_with_shared(_weights())), 16, 1)
    # + hs, hqs, shs, gate and the shared expert's 16 rows of y
    assert needs >= need + 16 * 64 * 3 + 16 * 8 + 16 * 64 * 2
    Ws = _with_shared(_weights())
    assert L.w8a8_moe_layer(ctypes.byref(Ws), FAKE, 1, 16, FAKE, FAKE, needs - 1, s) == WS_SMALL
    Ws.w_shared_gate = None
    assert L.w8a8_moe_layer(ctypes.byref(Ws), FAKE, 1, 16, FAKE, FAKE, needs, s) == INVALID
    Ws = _with_shared(_weights(), Is=0)
    assert L.w8a8_moe_layer(ctypes.byref(Ws), FAKE, 1, 16, FAKE, FAKE, needs, s) == INVALID
    Ws = _with_shared(_weights(), Is=48)
    assert L.w8a8_moe_layer(ctypes.byref(Ws), FAKE, 1, 16, FAKE, FAKE, needs, s) == SHAPE
    Ws = _with_shared(_weights(), ptr=MIS)
    assert L.w8a8_moe_layer(ctypes.byref(Ws), FAKE, 1, 16, FAKE, FAKE, needs, s) == ALIGN
    Ws = _with_shared(_weights())
    Ws.w4_gate_up = FAKE.value
    assert L.w8a8_moe_layer(ctypes.byref(Ws), FAKE, 1, 16, FAKE, FAKE, needs, s) == SHAPE
    # intermediates are laid out inside the workspace, in order, without overlap
    ptrs = (ctypes.c_void_p * 16)()
    base = 1 << 30
    assert L.w8a8_moe_layer_intermediates(ctypes.byref(W), 16, 1, ctypes.c_void_p(base), ptrs) == OK
    offs = [p - base for p in ptrs][:12]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs) and offs[-1] < need
    Ws = _with_shared(_weights())
    assert L.w8a8_moe_layer_intermediates(ctypes.byref(Ws), 16, 1, ctypes.c_void_p(base), ptrs) == OK
    offs = [p - base for p in ptrs]
    assert all(a < b for a, b in zip(offs, offs[1:])) and all(o % 256 == 0 for o in offs) and offs[-1] < needs
    big = _weights(E=128, k=8, H=4096, I=1536)
    assert L.w8a8_moe_layer_workspace_size(ctypes.byref(big), 8192, 0) > 8192 * 8 * 4096 * 2


def test_layer_rejects_router_offsets_beyond_32_bits(L):
    """The router kernels address token rows (T*H*4 bytes at most) and the
    router weight (E*H*2 bytes, E*H*4 for its fp32 copy) with 32-bit offsets:
    the layer returns SHAPE for larger inputs, as moe_route_topk does, instead
    of routing the far tokens wrongly."""
    s = None
    huge = 1 << 62
    W = _weights(E=8, k=1, H=4096, I=32)
    T = (1 << 31) // (4 * 4096) + 1            # T*H*4 just above 2^31, T*H below 2^31
    assert T * 4096 < (1 << 31)
    assert L.w8a8_moe_layer(ctypes.byref(W), FAKE, 0, T, FAKE, FAKE, huge, s) == SHAPE
    assert L.moe_route_topk(FAKE, 0, FAKE, T, 4096, 8, 1, 1, FAKE, FAKE, None, s) == SHAPE
    # one token below the bound passes the shape checks (the workspace check follows)
    assert L.w8a8_moe_layer(ctypes.byref(W), FAKE, 0, T - 2, FAKE, FAKE, 0, s) == WS_SMALL
    # the router weight: E*H*2 bytes fit, its fp32 copy's E*H*4 do not
    Wr = _weights(E=256, k=2, H=1 << 21, I=32)
    assert L.w8a8_moe_layer(ctypes.byref(Wr), FAKE, 0, 1, FAKE, FAKE, 0, s) == WS_SMALL
    Wr.w_gate_f32 = FAKE.value
    assert L.w8a8_moe_layer(ctypes.byref(Wr), FAKE, 0, 1, FAKE, FAKE, huge, s) == SHAPE


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(w8, "_lib", None)
    monkeypatch.setattr(w8, "LIB_PATH", "/nonexistent/libw8a8moe.so")
    with pytest.raises(ImportError):
        w8.lib()


def test_w4a8_entry_points_reject_before_launch(L):
    s = None
    assert L.w4a8_quant_weights(FAKE, 4, 40, FAKE, FAKE, FAKE, s) == SHAPE
    assert L.w4a8_quant_weights(FAKE, -1, 64, FAKE, FAKE, FAKE, s) == INVALID
    assert L.w4a8_quant_weights(MIS, 4, 64, FAKE, FAKE, FAKE, s) == ALIGN
    assert L.w4a8_quant_weights(FAKE, 0, 64, None, None, None, s) == OK
    # codes, then step-major scales and offsets, each part 256-byte aligned
    assert L.w4a8_packed_weights_size(2, 64, 300) == 2 * 2 * 3 * 2048 + 2 * 3 * 64 * 4 + 512
    assert L.w4a8_pack_weights(FAKE, FAKE, FAKE, 1, 40, 64, FAKE, s) == SHAPE
    assert L.w4a8_pack_weights(FAKE, FAKE, FAKE, 1, 64, 64, MIS, s) == ALIGN
    assert L.w4a8_pack_weights(FAKE, None, FAKE, 1, 64, 64, FAKE, s) == INVALID
    ws = L.w8a8_grouped_gemm_workspace_size(32, 64, 2)
    args = lambda **kw: dict(dict(A=FAKE, A_rows=32, a_scales=FAKE, gather=None, div=1, B=FAKE,
                                  off=FAKE, G=2, M=32, N=64, K=128, epi=1, od=0, out=FAKE, ws=FAKE, wsb=ws), **kw)
    call = lambda a: L.w4a8_grouped_gemm(a["A"], a["A_rows"], a["a_scales"], a["gather"], a["div"], a["B"],
                                         a["off"], a["G"], a["M"], a["N"], a["K"], a["epi"], a["od"],
                                         a["out"], a["ws"], a["wsb"], s)
    assert call(args(epi=0)) == INVALID            # no raw int32 sums across weight groups
    assert call(args(N=48, epi=2)) == SHAPE
    assert call(args(B=None)) == INVALID
    assert call(args(A=MIS)) == ALIGN
    assert call(args(wsb=ws - 1)) == WS_SMALL
    assert call(args(M=0, A=None, out=None, a_scales=None)) == OK


def test_linear_entry_points_reject_before_launch(L):
    s = None
    ws = L.w8a8_linear_workspace_size(64, 5120, 2048)
    assert ws >= 64 * 2048 + 64 * 4
    # a decode-sized linear with a long K splits it: int32 partial sums of the slices
    assert L.w8a8_linear_q_workspace_size(64, 2048, 4096) >= 2 * 64 * 2048 * 4
    assert L.w8a8_linear_q_workspace_size(64, 5120, 2048) == 0     # 16 steps: not worth a split
    assert L.w8a8_linear_q_workspace_size(4096, 2048, 4096) == 0   # enough tiles: no split
    assert L.w8a8_linear_workspace_size(64, 2048, 4096) >= 64 * 4096 + 64 * 4 + \
        L.w8a8_linear_q_workspace_size(64, 2048, 4096)
    lin = lambda **kw: (lambda a: L.w8a8_linear(a["x"], a["xd"], a["M"], a["K"], a["W"], a["sw"], a["N"], a["out"],
                                                a["od"], a["ws"], a["wsb"], s))(
        dict(dict(x=FAKE, xd=0, M=64, K=2048, W=FAKE, sw=FAKE, N=5120, out=FAKE, od=0, ws=FAKE, wsb=ws), **kw))
    assert lin(K=2040) == SHAPE
    assert lin(N=5112) == SHAPE
    assert lin(xd=3) == INVALID
    assert lin(od=2) == INVALID
    assert lin(W=None) == INVALID
    assert lin(x=MIS) == ALIGN
    assert lin(sw=MIS) == ALIGN
    assert lin(wsb=ws - 1) == WS_SMALL
    assert lin(M=0, x=None, out=None, ws=None, wsb=0) == OK
    assert lin(M=1 << 20, K=4096) == SHAPE   # M*K beyond 32-bit byte offsets
    qws = L.w8a8_linear_q_workspace_size(64, 2048, 4096)
    q = lambda **kw: (lambda a: L.w8a8_linear_q(a["xq"], a["sx"], a["M"], a["K"], a["W"], a["sw"], a["N"], a["out"],
                                                a["od"], a["ws"], a["wsb"], s))(
        dict(dict(xq=FAKE, sx=FAKE, M=64, K=4096, W=FAKE, sw=FAKE, N=2048, out=FAKE, od=1, ws=FAKE, wsb=qws), **kw))
    assert q(sx=None) == INVALID
    assert q(xq=MIS) == ALIGN
    assert q(ws=MIS) == ALIGN
    assert q(wsb=qws - 1) == WS_SMALL
    assert q(K=8) == SHAPE
    assert q(M=0, xq=None, sx=None, out=None) == OK

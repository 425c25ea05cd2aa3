"""W8A8 INT8 mixture-of-experts feed-forward layer for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libw8a8moe.so`` (declared in
``include/w8a8moe.h``).  This module only marshals arguments: it checks dtype,
device and contiguity, allocates outputs with torch, and passes raw device
pointers plus the current HIP stream.  Every computation runs in the HIP
kernels of the library; there is no CPU or PyTorch fallback, and every call
raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw8a8moe.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "w8a8moe.h")

BF16, F32, I32 = 0, 1, 2
B_ROWMAJOR, B_PACKED = 0, 1
EPI_RAW_I32, EPI_DEQUANT, EPI_DEQUANT_SWIGLU = 0, 1, 2
LAYER_STAGES = 7
STAGE_NAMES = ("route", "quant_x", "permute", "gate_up_gemm", "quant_h", "down_gemm", "combine")
INTERMEDIATES = ("ids", "w", "xq", "sx", "offsets", "sorted_pair", "pair_pos", "h", "hq", "sh", "y", "y_exp",
                 "hs", "hqs", "shs", "gate")


class W8A8Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


class _Weights(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("k", ctypes.c_int), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("w_gate", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("s_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p), ("w_gate_f32", ctypes.c_void_p),
                ("w4_gate_up", ctypes.c_void_p), ("I_shared", ctypes.c_int64),
                ("w_shared_gate_up", ctypes.c_void_p), ("s_shared_gate_up", ctypes.c_void_p),
                ("w_shared_down", ctypes.c_void_p), ("s_shared_down", ctypes.c_void_p),
                ("w_shared_gate", ctypes.c_void_p), ("w_gate_packed", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libw8a8moe.so (built by ``w8a8_int8_quantized_bf16_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libw8a8moe.so is not built (run w8a8_int8_quantized_bf16_amd.build.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.w8a8_status_string.argtypes = [i32]
    L.w8a8_status_string.restype = ctypes.c_char_p
    L.w8a8_quant_act.argtypes = [P, i32, i64, i64, i64, P, P, P]
    L.moe_route_topk.argtypes = [P, i32, P, i64, i64, i32, i32, i32, P, P, P, P]
    L.moe_route_topk_packed.argtypes = [P, i32, P, P, i64, i64, i32, i32, i32, P, P, P, P]
    L.moe_router_widen.argtypes = [P, i32, i64, P, P]
    L.moe_router_pack.argtypes = [P, i32, i64, P, P]
    L.w8a8_linear_workspace_size.argtypes = [i64, i64, i64]
    L.w8a8_linear_workspace_size.restype = sz
    L.w8a8_linear_q_workspace_size.argtypes = [i64, i64, i64]
    L.w8a8_linear_q_workspace_size.restype = sz
    L.w8a8_linear.argtypes = [P, i32, i64, i64, P, P, i64, P, i32, P, sz, P]
    L.w8a8_linear_q.argtypes = [P, P, i64, i64, P, P, i64, P, i32, P, sz, P]
    L.moe_permute_workspace_size.argtypes = [i64, i32, i32]
    L.moe_permute_workspace_size.restype = sz
    L.moe_permute.argtypes = [P, i64, i32, i32, P, P, P, P, sz, P]
    L.w8a8_grouped_gemm_workspace_size.argtypes = [i64, i64, i32]
    L.w8a8_grouped_gemm_workspace_size.restype = sz
    L.w8a8_grouped_gemm.argtypes = [P, i64, P, P, i32, P, i32, P, P, i32, i64, i64, i64, i32, i32, P, P, sz, P]
    L.w8a8_grouped_gemm_noalloc.argtypes = [P, i64, P, P, i32, P, i32, P, P, i32, i64, i64, i64, i32, i32, P, P]
    L.w8a8_packed_weights_size.argtypes = [i32, i64, i64]
    L.w8a8_packed_weights_size.restype = sz
    L.w8a8_pack_weights.argtypes = [P, i32, i64, i64, P, P]
    L.moe_combine.argtypes = [P, i32, P, P, i64, i32, i64, P, i32, P]
    L.w4a8_quant_weights.argtypes = [P, i64, i64, P, P, P, P]
    L.w4a8_packed_weights_size.argtypes = [i32, i64, i64]
    L.w4a8_packed_weights_size.restype = sz
    L.w4a8_pack_weights.argtypes = [P, P, P, i32, i64, i64, P, P]
    L.w4a8_grouped_gemm.argtypes = [P, i64, P, P, i32, P, P, i32, i64, i64, i64, i32, i32, P, P, sz, P]
    WP = ctypes.POINTER(_Weights)
    L.w8a8_moe_layer_workspace_size.argtypes = [WP, i64, i32]
    L.w8a8_moe_layer_workspace_size.restype = sz
    L.w8a8_moe_layer.argtypes = [WP, P, i32, i64, P, P, sz, P]
    L.w8a8_moe_layer_events.argtypes = [WP, P, i32, i64, P, P, sz, P, ctypes.POINTER(P), i32]
    L.w8a8_moe_layer_intermediates.argtypes = [WP, i64, i32, P, ctypes.POINTER(P)]
    for name in ("w8a8_quant_act", "moe_route_topk", "moe_permute", "w8a8_grouped_gemm", "moe_combine",
                 "w8a8_pack_weights", "w4a8_quant_weights", "w4a8_pack_weights", "w4a8_grouped_gemm",
                 "w8a8_moe_layer", "w8a8_moe_layer_events", "w8a8_moe_layer_intermediates"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def header_functions():
    """Names of the functions declared in include/w8a8moe.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_\w+|w4a8_\w+|moe_\w+)\s*\(", text)))


def status_string(status):
    return lib().w8a8_status_string(int(status)).decode()


def _check(rc, where):
    if rc != 0:
        raise W8A8Error(rc, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev=None):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _act_dtype(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("expected bfloat16 or float32, got %s" % t.dtype)


def _torch_dtype(code):
    return {BF16: torch.bfloat16, F32: torch.float32, I32: torch.int32}[code]


def _need(t, name, dtype=None, dim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if dim is not None and t.dim() != dim:
        raise ValueError("%s must have %d dims" % (name, dim))


# ------------------------------------------------------------------ stages ---

def quant_act(x):
    """Per-row symmetric int8 quantisation: returns (codes int8 [rows, cols], scales fp32 [rows])."""
    _need(x, "x", dim=2)
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().w8a8_quant_act(_p(x), _act_dtype(x), rows, cols, cols, _p(q), _p(s), _stream(x.device)),
           "w8a8_quant_act")
    return q, s


def route_topk(x, w_gate, k, renormalize=True, return_logits=False, w_gate_packed=None):
    """Router: (ids int32 [T,k], weights fp32 [T,k][, logits fp32 [T,E]]).
    w_gate_packed: optional router_pack() copy of w_gate (same results)."""
    _need(x, "x", dim=2)
    _need(w_gate, "w_gate", torch.bfloat16, 2)
    T, H = x.shape
    E = w_gate.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if return_logits else None
    if w_gate_packed is None:
        _check(lib().moe_route_topk(_p(x), _act_dtype(x), _p(w_gate), T, H, E, k, int(bool(renormalize)), _p(ids),
                                    _p(w), _p(logits), _stream(x.device)), "moe_route_topk")
    else:
        _need(w_gate_packed, "w_gate_packed", torch.bfloat16, 3)
        _check(lib().moe_route_topk_packed(_p(x), _act_dtype(x), _p(w_gate), _p(w_gate_packed), T, H, E, k,
                                           int(bool(renormalize)), _p(ids), _p(w), _p(logits), _stream(x.device)),
               "moe_route_topk_packed")
    return (ids, w, logits) if return_logits else (ids, w)


def permute(ids, E):
    """Stable grouping of pairs by expert: (offsets [E+1], sorted_pair [P], pair_pos [P]) int32."""
    _need(ids, "ids", torch.int32, 2)
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    nws = max(int(lib().moe_permute_workspace_size(T, k, E)), 256)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    _check(lib().moe_permute(_p(ids), T, k, E, _p(offsets), _p(sp), _p(pos), _p(ws), nws, _stream(dev)),
           "moe_permute")
    return offsets, sp, pos


def pack_weights(B):
    """Re-lay int8 weights [G, N, K] into the packed MFMA-fragment layout (uint8 bytes)."""
    _need(B, "B", torch.int8, 3)
    G, N, K = B.shape
    n = int(lib().w8a8_packed_weights_size(G, N, K))
    out = torch.empty(n, dtype=torch.int8, device=B.device)
    _check(lib().w8a8_pack_weights(_p(B), G, N, K, _p(out), _stream(B.device)), "w8a8_pack_weights")
    return out


def linear(x, w_packed, w_scales, N, out_dtype=BF16, ws=None, out=None):
    """Dense W8A8 linear: x [M,K] bf16/fp32 quantised per row, times the packed
    int8 weights (pack_weights of [N,K] codes) with per-channel scales w_scales
    [N]; out [M,N]."""
    _need(x, "x", dim=2)
    _need(w_packed, "w_packed", torch.int8)
    _need(w_scales, "w_scales", torch.float32, 1)
    M, K = x.shape
    if ws is None:
        ws = torch.empty(max(int(lib().w8a8_linear_workspace_size(M, N, K)), 256), dtype=torch.uint8,
                         device=x.device)
    if out is None:
        out = torch.empty((M, N), dtype=_torch_dtype(out_dtype), device=x.device)
    _check(lib().w8a8_linear(_p(x), _act_dtype(x), M, K, _p(w_packed), _p(w_scales), N, _p(out), out_dtype, _p(ws),
                             ws.numel(), _stream(x.device)), "w8a8_linear")
    return out


def linear_q(xq, x_scales, w_packed, w_scales, N, out_dtype=BF16, out=None, split=True):
    """The dense W8A8 linear on rows already quantised (xq int8 [M,K], x_scales
    [M]); split=False runs it without splitting K (no workspace)."""
    _need(xq, "xq", torch.int8, 2)
    _need(x_scales, "x_scales", torch.float32, 1)
    M, K = xq.shape
    if out is None:
        out = torch.empty((M, N), dtype=_torch_dtype(out_dtype), device=xq.device)
    nws = int(lib().w8a8_linear_q_workspace_size(M, N, K)) if split else 0
    ws = torch.empty(nws, dtype=torch.uint8, device=xq.device) if nws else None
    _check(lib().w8a8_linear_q(_p(xq), _p(x_scales), M, K, _p(w_packed), _p(w_scales), N, _p(out), out_dtype,
                               _p(ws), nws, _stream(xq.device)), "w8a8_linear_q")
    return out


def grouped_gemm(A, a_scales, gather, gather_div, B, b_scales, offsets, epilogue, out_dtype=BF16, M_total=None,
                 b_shape=None):
    """Grouped W8A8 GEMM (see include/w8a8moe.h).  B is [G, N, K] int8, or the
    1-D packed bytes of pack_weights() with b_shape=(G, N, K)."""
    _need(A, "A", torch.int8, 2)
    _need(B, "B", torch.int8)
    _need(offsets, "offsets", torch.int32, 1)
    if b_shape is None:
        if B.dim() != 3:
            raise ValueError("B must be [G, N, K] unless b_shape is given for packed weights")
        G, N, K = B.shape
        layout = B_ROWMAJOR
    else:
        G, N, K = b_shape
        layout = B_PACKED
    if M_total is None:
        M_total = gather.shape[0] if gather is not None else A.shape[0]
    if epilogue == EPI_RAW_I32:
        out_dtype = I32
        out = torch.empty((M_total, N), dtype=torch.int32, device=A.device)
    else:
        ncol = N if epilogue == EPI_DEQUANT else N // 2
        out = torch.empty((M_total, ncol), dtype=_torch_dtype(out_dtype), device=A.device)
    nws = int(lib().w8a8_grouped_gemm_workspace_size(M_total, N, G))
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=A.device)
    _check(lib().w8a8_grouped_gemm(_p(A), A.shape[0], _p(a_scales), _p(gather), int(gather_div), _p(B), layout,
                                   _p(b_scales), _p(offsets), G, M_total, N, K, epilogue, out_dtype, _p(out),
                                   _p(ws), ws.numel(), _stream(A.device)), "w8a8_grouped_gemm")
    return out


W4_GROUP = 128


def w4a8_quant_weights(w):
    """W4 codes of fp32 weights [rows, cols]: (codes int8 [rows, cols] in [-8, 7],
    scales fp32 [rows, ceil(cols/128)], offsets int8 [rows, ceil(cols/128)])."""
    _need(w, "w", torch.float32, 2)
    rows, cols = w.shape
    ng = (cols + W4_GROUP - 1) // W4_GROUP
    q = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    s = torch.empty((rows, ng), dtype=torch.float32, device=w.device)
    o = torch.empty((rows, ng), dtype=torch.int8, device=w.device)
    _check(lib().w4a8_quant_weights(_p(w), rows, cols, _p(q), _p(s), _p(o), _stream(w.device)), "w4a8_quant_weights")
    return q, s, o


def w4a8_pack_weights(q, scales, offsets):
    """Pack W4 codes [G, N, K] two per byte in the W4A8 GEMM layout, followed
    by their group scales and offsets ([G, N, ceil(K/128)]) re-laid step-major
    (uint8 bytes)."""
    _need(q, "q", torch.int8, 3)
    _need(scales, "scales", torch.float32)
    _need(offsets, "offsets", torch.int8)
    G, N, K = q.shape
    n = int(lib().w4a8_packed_weights_size(G, N, K))
    out = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(lib().w4a8_pack_weights(_p(q), _p(scales), _p(offsets), G, N, K, _p(out), _stream(q.device)),
           "w4a8_pack_weights")
    return out


def w4a8_grouped_gemm(A, a_scales, gather, gather_div, B_packed, offsets, epilogue, out_dtype=BF16, M_total=None,
                      b_shape=None):
    """Grouped W4A8 GEMM: B_packed from w4a8_pack_weights of codes of shape
    b_shape = (G, N, K) with their scales and offsets."""
    _need(A, "A", torch.int8, 2)
    _need(B_packed, "B_packed", torch.uint8, 1)
    _need(offsets, "offsets", torch.int32, 1)
    G, N, K = b_shape
    if M_total is None:
        M_total = gather.shape[0] if gather is not None else A.shape[0]
    ncol = N if epilogue == EPI_DEQUANT else N // 2
    out = torch.empty((M_total, ncol), dtype=_torch_dtype(out_dtype), device=A.device)
    nws = int(lib().w8a8_grouped_gemm_workspace_size(M_total, N, G))
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=A.device)
    _check(lib().w4a8_grouped_gemm(_p(A), A.shape[0], _p(a_scales), _p(gather), int(gather_div), _p(B_packed),
                                   _p(offsets), G, M_total, N, K, epilogue, out_dtype, _p(out), _p(ws), ws.numel(),
                                   _stream(A.device)), "w4a8_grouped_gemm")
    return out


def combine(y, w, pair_pos, out_dtype=None):
    """out[t] = sum_j w[t,j] * y[pair_pos[t*k+j]]."""
    _need(y, "y", dim=2)
    _need(w, "w", torch.float32, 2)
    _need(pair_pos, "pair_pos", torch.int32, 1)
    T, k = w.shape
    H = y.shape[1]
    od = _act_dtype(y) if out_dtype is None else out_dtype
    out = torch.empty((T, H), dtype=_torch_dtype(od), device=y.device)
    _check(lib().moe_combine(_p(y), _act_dtype(y), _p(w), _p(pair_pos), T, k, H, _p(out), od, _stream(y.device)),
           "moe_combine")
    return out


# ------------------------------------------------------------------- layer ---

def router_widen(w_gate):
    """The bf16 router weight widened to fp32 (exact) by the library."""
    _need(w_gate, "w_gate", torch.bfloat16, 2)
    E, H = w_gate.shape
    out = torch.empty((E, H), dtype=torch.float32, device=w_gate.device)
    _check(lib().moe_router_widen(_p(w_gate), E, H, _p(out), _stream()), "moe_router_widen")
    return out


def router_pack(w_gate):
    """The bf16 router weight re-laid [H/8][E][8] by the library (a copy)."""
    _need(w_gate, "w_gate", torch.bfloat16, 2)
    E, H = w_gate.shape
    out = torch.empty((H // 8, E, 8), dtype=torch.bfloat16, device=w_gate.device)
    _check(lib().moe_router_pack(_p(w_gate), E, H, _p(out), _stream()), "moe_router_pack")
    return out


class MoEWeights:
    """Device tensors of one layer.
    w_gate [E,H] bf16; w_gate_up [E,2I,H] int8 codes (gate rows, then up rows);
    s_gate_up [E,2I] fp32; w_down [E,H,I] int8 codes; s_down [E,H] fp32.
    The layer reads the codes in the packed layout (pack_weights), built here."""

    def __init__(self, w_gate, w_gate_up, s_gate_up, w_down, s_down, k, w4=None, shared=None):
        """w4: optional W4A8 gate_up_proj (codes [E,2I,H], scales and offsets
        [E,2I,ceil(H/128)]), used instead of w_gate_up / s_gate_up (which may
        then be None).  shared: optional shared expert, a tuple (gate_up codes
        [2Is,H] int8, scales [2Is] fp32, down codes [H,Is] int8, scales [H]
        fp32, shared_expert_gate [H] bf16)."""
        _need(w_gate, "w_gate", torch.bfloat16, 2)
        _need(w_down, "w_down", torch.int8, 3)
        _need(s_down, "s_down", torch.float32, 2)
        if w4 is None:
            _need(w_gate_up, "w_gate_up", torch.int8, 3)
            _need(s_gate_up, "s_gate_up", torch.float32, 2)
            E, twoI, H = w_gate_up.shape
        else:
            _need(w4[0], "w4 codes", torch.int8, 3)
            E, twoI, H = w4[0].shape
        self.E, self.H, self.I, self.k = E, H, twoI // 2, int(k)
        self.tensors = (w_gate, w_gate_up, s_gate_up, w_down, s_down)
        self.w_gate, self.w_gate_up, self.s_gate_up, self.w_down, self.s_down = self.tensors
        self.w4 = w4
        self.p_gate_up = pack_weights(w_gate_up) if w_gate_up is not None else None
        self.p_down = pack_weights(w_down)
        self.w_gate_f32 = router_widen(w_gate)
        self.w_gate_packed = router_pack(w_gate)
        self.p4_gate_up = w4a8_pack_weights(*w4) if w4 is not None else None
        self.shared = shared
        self.Is = 0
        sp = (None,) * 5
        if shared is not None:
            sgu, ssgu, sdn, ssd, wsg = shared
            _need(sgu, "shared gate_up", torch.int8, 2)
            _need(ssgu, "shared gate_up scales", torch.float32, 1)
            _need(sdn, "shared down", torch.int8, 2)
            _need(ssd, "shared down scales", torch.float32, 1)
            _need(wsg, "shared_expert_gate", torch.bfloat16, 1)
            self.Is = sgu.shape[0] // 2
            self.p_shared = (pack_weights(sgu[None]), pack_weights(sdn[None]))
            sp = (self.p_shared[0], ssgu, self.p_shared[1], ssd, wsg)
        ptr = lambda t: None if t is None else t.data_ptr()
        self.c = _Weights(E, self.k, H, self.I, w_gate.data_ptr(), ptr(self.p_gate_up), ptr(s_gate_up),
                          self.p_down.data_ptr(), s_down.data_ptr(), self.w_gate_f32.data_ptr(),
                          ptr(self.p4_gate_up), self.Is, *[ptr(t) for t in sp], self.w_gate_packed.data_ptr())

    @classmethod
    def quantize(cls, w_gate, gate_up_f32, down_f32, k, w4=False, shared=None):
        """Static quantisation of fp32 expert weights on the GPU: per output
        channel int8 (the same row kernel as the activations), or with w4=True
        W4A8 gate_up_proj (groups of 128) and int8 down_proj.  shared: optional
        (gate_up fp32 [2Is,H], down fp32 [H,Is], shared_expert_gate bf16 [H]),
        quantised per output channel to int8 (the gate stays bf16)."""
        E, twoI, H = gate_up_f32.shape
        qd, sd = quant_act(down_f32.reshape(E * H, twoI // 2))
        se = None
        if shared is not None:
            sgu_f, sdn_f, wsg = shared
            qsgu, ssgu = quant_act(sgu_f)
            qsdn, ssdn = quant_act(sdn_f)
            se = (qsgu, ssgu, qsdn, ssdn, wsg)
        if w4:
            q4, s4, o4 = w4a8_quant_weights(gate_up_f32.reshape(E * twoI, H))
            return cls(w_gate, None, None, qd.view(E, H, twoI // 2), sd.view(E, H), k,
                       w4=(q4.view(E, twoI, H), s4.view(E, twoI, -1), o4.view(E, twoI, -1)), shared=se)
        qgu, sgu = quant_act(gate_up_f32.reshape(E * twoI, H))
        return cls(w_gate, qgu.view(E, twoI, H), sgu.view(E, twoI), qd.view(E, H, twoI // 2), sd.view(E, H), k,
                   shared=se)


def moe_layer_workspace_size(W: MoEWeights, T, x_dtype=BF16):
    return int(lib().w8a8_moe_layer_workspace_size(ctypes.byref(W.c), T, x_dtype))


def moe_layer_workspace(W: MoEWeights, T, x_dtype=BF16, device="cuda"):
    return torch.empty(max(moe_layer_workspace_size(W, T, x_dtype), 256), dtype=torch.uint8, device=device)


def moe_layer(W: MoEWeights, x, ws=None, out=None, events=None):
    """The W8A8 MoE layer: out [T,H] in the dtype of x."""
    _need(x, "x", dim=2)
    T, H = x.shape
    dt = _act_dtype(x)
    if ws is None:
        ws = moe_layer_workspace(W, T, dt, x.device)
    if out is None:
        out = torch.empty_like(x)
    if events is None:
        rc = lib().w8a8_moe_layer(ctypes.byref(W.c), _p(x), dt, T, _p(out), _p(ws), ws.numel(), _stream(x.device))
    else:
        # None skips a mark; a torch event must have been recorded once (torch
        # creates the HIP event lazily)
        if any(e is not None and e.cuda_event == 0 for e in events):
            raise ValueError("events must have been recorded once (torch creates the HIP event lazily)")
        arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(None if e is None else e.cuda_event)
                                                  for e in events])
        rc = lib().w8a8_moe_layer_events(ctypes.byref(W.c), _p(x), dt, T, _p(out), _p(ws), ws.numel(),
                                         _stream(x.device), arr, len(events))
    _check(rc, "w8a8_moe_layer")
    return out


def moe_layer_intermediates(W: MoEWeights, T, ws, x_dtype=BF16):
    """Views into `ws` of the intermediate results of the last layer call."""
    ptrs = (ctypes.c_void_p * len(INTERMEDIATES))()
    _check(lib().w8a8_moe_layer_intermediates(ctypes.byref(W.c), T, x_dtype, _p(ws), ptrs),
           "w8a8_moe_layer_intermediates")
    P, E, H, I = T * W.k, W.E, W.H, W.I
    Ts, Is = (T, W.Is) if W.Is else (0, 0)
    spec = dict(ids=((T, W.k), torch.int32), w=((T, W.k), torch.float32), xq=((T, H), torch.int8),
                sx=((T,), torch.float32), offsets=((E + 1,), torch.int32), sorted_pair=((P,), torch.int32),
                pair_pos=((P,), torch.int32), h=((P, I), torch.bfloat16), hq=((P, I), torch.int8),
                sh=((P,), torch.float32), y=((P + Ts, H), torch.int16),
                y_exp=((P + Ts, (H + 63) // 64), torch.int8), hs=((Ts, Is), torch.bfloat16),
                hqs=((Ts, Is), torch.int8), shs=((Ts,), torch.float32), gate=((Ts,), torch.float32))
    base = ws.data_ptr()
    out = {}
    for name, p in zip(INTERMEDIATES, ptrs):
        shape, dtype = spec[name]
        off = p - base
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        out[name] = ws[off:off + nbytes].view(dtype).view(shape)
    return out

"""CPU oracle for the W8A8 INT8 MoE feed-forward layer -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never uses it, and it
imports nothing from the GPU package.

The arithmetic lives in ``oracle.c`` (plain C loops, built with
``-O2 -ffp-contract=off``, no fast-math).  This module only builds that file
with gcc and marshals numpy arrays into it.  bf16 arrays are passed as their
uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16, F32 = 0, 1
RAW_I32, DEQUANT, DEQUANT_SWIGLU = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_quant_rows.argtypes = [P, i32, i64, i64, i64, P, P]
        L.oracle_route_topk.argtypes = [P, i32, P, i64, i64, i32, i32, i32, P, P, P]
        L.oracle_route_topk_chunked.argtypes = [P, i32, P, i64, i64, i32, i32, i32, P, P, P, i64]
        L.oracle_permute.argtypes = [P, i64, i32, i32, P, P, P]
        L.oracle_grouped_gemm.argtypes = [P, P, P, i32, P, P, P, i32, i64, i64, i32, i32, P]
        L.oracle_combine.argtypes = [P, i32, P, P, i64, i32, i64, P, i32]
        L.oracle_moe_layer.argtypes = [P, i32, i64, i64, i32, i32, i64, P, P, P, P, P, P] + [P] * 12
        L.oracle_moe_layer_tokens.argtypes = [P, i32, i64, i32, i32, i64, P, P, P, P, P, P, i64, P]
        L.oracle_quant_w4_rows.argtypes = [P, i64, i64, P, P, P]
        L.oracle_w4a8_grouped_gemm.argtypes = [P, P, P, i32, P, P, P, P, i32, i64, i64, i32, i32, P]
        L.oracle_moe_layer_w4.argtypes = [P, i32, i64, i64, i32, i32, i64, P, P, P, P, P, P, P] + [P] * 10
        L.oracle_moe_layer_w4_tokens.argtypes = [P, i32, i64, i32, i32, i64, P, P, P, P, P, P, P, i64, P]
        L.oracle_moe_layer_shared.argtypes = ([P, i32, i64, i64, i32, i32, i64, P, P, P, P, P, i64, P, P, P, P, P, P]
                                              + [P] * 15)
        L.oracle_moe_layer_shared_tokens.argtypes = [P, i32, i64, i32, i32, i64, P, P, P, P, P, i64, P, P, P, P, P,
                                                     P, i64, P]
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_f64_to_bf16.argtypes = [d]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = d
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _xdtype(x):
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return F32
    raise TypeError("x must be bf16 bits (uint16) or float32, got %s" % x.dtype)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's loops over independent rows (results do not
    depend on it)."""
    lib().oracle_set_num_threads(int(n))


def f64_to_bf16(v: float) -> int:
    return int(lib().oracle_f64_to_bf16(float(v)))


def bf16_to_f64(b: int) -> float:
    return float(lib().oracle_bf16_to_f64(int(b)))


def quant_rows(x):
    """Per-row symmetric int8 quantisation. x [rows, cols] bf16 bits or fp32."""
    x = np.ascontiguousarray(x)
    dt = _xdtype(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    lib().oracle_quant_rows(_p(x), dt, rows, cols, cols, _p(q), _p(s))
    return q, s


ROUTE_CHUNK = 512   # R6: hidden indices per fma chain of a router score


def route_topk(x, wg, k, renormalize=True, chunk=ROUTE_CHUNK):
    """Router: returns ids [T,k] int32, w [T,k] fp32, logits [T,E] fp32.
    chunk: hidden indices per fma chain (R6's 512; 0 for one chain over all
    of H, a study of how the order moves the selection, not the layer's)."""
    x = np.ascontiguousarray(x)
    wg = _c(wg, np.uint16)
    T, H = x.shape
    E = wg.shape[0]
    assert wg.shape[1] == H
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    logits = np.empty((T, E), np.float32)
    lib().oracle_route_topk_chunked(_p(x), _xdtype(x), _p(wg), T, H, E, k, int(bool(renormalize)),
                                    _p(ids), _p(w), _p(logits), int(chunk))
    return ids, w, logits


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, np.int32)
    sorted_pair = np.empty(T * k, np.int32)
    pair_pos = np.empty(T * k, np.int32)
    lib().oracle_permute(_p(ids), T, k, E, _p(offsets), _p(sorted_pair), _p(pair_pos))
    return offsets, sorted_pair, pair_pos


def grouped_gemm(A, a_scales, gather, gather_div, B, b_scales, offsets, epilogue, out_dtype=BF16):
    """Grouped W8A8 GEMM (see oracle.c).  Returns the output array."""
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    offsets = _c(offsets, np.int32)
    G, N, K = B.shape
    M = int(offsets[-1])
    a_scales = None if a_scales is None else _c(a_scales, np.float32)
    b_scales = None if b_scales is None else _c(b_scales, np.float32)
    gather = None if gather is None else _c(gather, np.int32)
    if epilogue == RAW_I32:
        out = np.empty((M, N), np.int32)
    else:
        ncol = N if epilogue == DEQUANT else N // 2
        out = np.empty((M, ncol), np.uint16 if out_dtype == BF16 else np.float32)
    lib().oracle_grouped_gemm(_p(A), _p(a_scales), _p(gather), int(gather_div), _p(B), _p(b_scales),
                              _p(offsets), G, N, K, epilogue, out_dtype, _p(out))
    return out


def combine(y, w, pair_pos, out_dtype):
    """y [T*k, H] as bf16 bits, fp32 or fp64; w [T,k]; pair_pos [T*k]."""
    y = np.ascontiguousarray(y)
    ydt = {np.dtype(np.uint16): 0, np.dtype(np.float32): 1, np.dtype(np.float64): 2}[y.dtype]
    w = _c(w, np.float32)
    pair_pos = _c(pair_pos, np.int32)
    T, k = w.shape
    H = y.shape[1]
    out = np.empty((T, H), np.uint16 if out_dtype == BF16 else np.float32)
    lib().oracle_combine(_p(y), ydt, _p(w), _p(pair_pos), T, k, H, _p(out), out_dtype)
    return out


def moe_layer(x, wg, wgu, sgu, wd, sd, k, intermediates=False):
    """Whole W8A8 MoE layer.  x [T,H] bf16 bits or fp32; wg [E,H] bf16 bits;
    wgu [E,2I,H] int8, sgu [E,2I] fp32; wd [E,H,I] int8, sd [E,H] fp32.
    Returns out [T,H] (dtype of x) and, with intermediates=True, a dict of every
    intermediate result."""
    x = np.ascontiguousarray(x)
    dt = _xdtype(x)
    wg = _c(wg, np.uint16)
    wgu = _c(wgu, np.int8)
    wd = _c(wd, np.int8)
    sgu = _c(sgu, np.float32)
    sd = _c(sd, np.float32)
    T, H = x.shape
    E, twoI, H2 = wgu.shape
    I = twoI // 2
    assert H2 == H and wd.shape == (E, H, I) and wg.shape == (E, H)
    P = T * k
    out = np.empty((T, H), x.dtype)
    inter = {}
    if intermediates:
        inter = dict(
            ids=np.empty((T, k), np.int32), w=np.empty((T, k), np.float32),
            xq=np.empty((T, H), np.int8), sx=np.empty(T, np.float32),
            offsets=np.empty(E + 1, np.int32), sorted_pair=np.empty(P, np.int32),
            pair_pos=np.empty(P, np.int32), acc_gu=np.empty((P, 2 * I), np.int32),
            h=np.empty((P, I), np.uint16), hq=np.empty((P, I), np.int8),
            sh=np.empty(P, np.float32), acc_d=np.empty((P, H), np.int32))
    g = inter.get
    lib().oracle_moe_layer(_p(x), dt, T, H, E, k, I, _p(wg), _p(wgu), _p(sgu), _p(wd), _p(sd), _p(out),
                           _p(g("ids")), _p(g("w")), _p(g("xq")), _p(g("sx")), _p(g("offsets")),
                           _p(g("sorted_pair")), _p(g("pair_pos")), _p(g("acc_gu")), _p(g("h")),
                           _p(g("hq")), _p(g("sh")), _p(g("acc_d")))
    return (out, inter) if intermediates else out


def moe_layer_tokens(x, wg, wgu, sgu, wd, sd, k, tokens):
    """Rows `tokens` of the layer output (the layer couples no tokens)."""
    x = np.ascontiguousarray(x)
    dt = _xdtype(x)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    E, twoI, H = wgu.shape
    I = twoI // 2
    out = np.empty((len(tok), H), x.dtype)
    lib().oracle_moe_layer_tokens(_p(x), dt, H, E, k, I, _p(_c(wg, np.uint16)), _p(_c(wgu, np.int8)),
                                  _p(_c(sgu, np.float32)), _p(_c(wd, np.int8)), _p(_c(sd, np.float32)),
                                  _p(tok), len(tok), _p(out))
    return out


def bf16_bits_to_f32(b):
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------- W4A8 ---

W4_GROUP = 128


def quant_w4_rows(w):
    """W4 codes of fp32 weights [rows, cols] (R17): (codes int8 [rows, cols] in
    [-8, 7], scales fp32 [rows, ceil(cols/128)], offsets int8 [rows, ceil(cols/128)])."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    ng = (cols + W4_GROUP - 1) // W4_GROUP
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows, ng), np.float32)
    o = np.empty((rows, ng), np.int8)
    lib().oracle_quant_w4_rows(_p(w), rows, cols, _p(q), _p(s), _p(o))
    return q, s, o


def w4a8_grouped_gemm(A, a_scales, gather, gather_div, Bq, b_scales, b_offs, offsets, epilogue, out_dtype=BF16):
    """Grouped W4A8 GEMM (epilogue DEQUANT or DEQUANT_SWIGLU): Bq [G,N,K] codes,
    b_scales / b_offs [G,N,ceil(K/128)]."""
    A = _c(A, np.int8)
    Bq = _c(Bq, np.int8)
    a_scales = _c(a_scales, np.float32)
    b_scales = _c(b_scales, np.float32)
    b_offs = _c(b_offs, np.int8)
    offsets = _c(offsets, np.int32)
    G, N, K = Bq.shape
    M = int(offsets[-1]) if gather is None else len(gather)
    gather = None if gather is None else _c(gather, np.int32)
    ncol = N if epilogue == DEQUANT else N // 2
    out = np.empty((M, ncol), np.uint16 if out_dtype == BF16 else np.float32)
    lib().oracle_w4a8_grouped_gemm(_p(A), _p(a_scales), _p(gather), int(gather_div), _p(Bq), _p(b_scales),
                                   _p(b_offs), _p(offsets), G, N, K, epilogue, out_dtype, _p(out))
    return out


def moe_layer_w4(x, wg, wgu4, sgu4, ogu4, wd, sd, k, intermediates=False):
    """The layer with W4A8 gate_up weights (codes [E,2I,H], scales / offsets
    [E,2I,ceil(H/128)]) and W8A8 down weights."""
    x = np.ascontiguousarray(x)
    dt = _xdtype(x)
    wgu4 = _c(wgu4, np.int8)
    E, twoI, H = wgu4.shape
    I = twoI // 2
    T = x.shape[0]
    P = T * k
    out = np.empty((T, H), x.dtype)
    inter = {}
    if intermediates:
        inter = dict(
            ids=np.empty((T, k), np.int32), w=np.empty((T, k), np.float32),
            xq=np.empty((T, H), np.int8), sx=np.empty(T, np.float32),
            offsets=np.empty(E + 1, np.int32), sorted_pair=np.empty(P, np.int32),
            pair_pos=np.empty(P, np.int32), h=np.empty((P, I), np.uint16), hq=np.empty((P, I), np.int8),
            sh=np.empty(P, np.float32))
    g = inter.get
    lib().oracle_moe_layer_w4(_p(x), dt, T, H, E, k, I, _p(_c(wg, np.uint16)), _p(wgu4),
                              _p(_c(sgu4, np.float32)), _p(_c(ogu4, np.int8)), _p(_c(wd, np.int8)),
                              _p(_c(sd, np.float32)), _p(out),
                              _p(g("ids")), _p(g("w")), _p(g("xq")), _p(g("sx")), _p(g("offsets")),
                              _p(g("sorted_pair")), _p(g("pair_pos")), _p(g("h")), _p(g("hq")), _p(g("sh")))
    return (out, inter) if intermediates else out


def moe_layer_w4_tokens(x, wg, wgu4, sgu4, ogu4, wd, sd, k, tokens):
    """Rows `tokens` of the W4A8-gate_up layer output."""
    x = np.ascontiguousarray(x)
    dt = _xdtype(x)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    E, twoI, H = wgu4.shape
    I = twoI // 2
    out = np.empty((len(tok), H), x.dtype)
    lib().oracle_moe_layer_w4_tokens(_p(x), dt, H, E, k, I, _p(_c(wg, np.uint16)), _p(_c(wgu4, np.int8)),
                                     _p(_c(sgu4, np.float32)), _p(_c(ogu4, np.int8)), _p(_c(wd, np.int8)),
                                     _p(_c(sd, np.float32)), _p(tok), len(tok), _p(out))
    return out


# ---------------------------------------------------------- shared expert ---


def _shared_args(se, H):
    """(Is, codes/scales of gate_up and down, gate bits) of a shared expert dict
    {wgu [2Is,H] int8, sgu [2Is] fp32, wd [H,Is] int8, sd [H] fp32, wsg [H] bf16 bits}."""
    wgu = _c(se["wgu"], np.int8)
    twoIs, H2 = wgu.shape
    Is = twoIs // 2
    wd = _c(se["wd"], np.int8)
    assert H2 == H and wd.shape == (H, Is) and np.shape(se["wsg"]) == (H,)
    return Is, (wgu, _c(se["sgu"], np.float32), wd, _c(se["sd"], np.float32), _c(se["wsg"], np.uint16))


def moe_layer_shared(x, wg, wgu, sgu, wd, sd, k, shared, intermediates=False):
    """The layer with a shared expert (R18, R19); `shared` as in _shared_args.
    Intermediates: the routed ones (ids, w, xq, sx, offsets, sorted_pair,
    pair_pos, h, hq, sh) and the shared expert's gate [T] (fp64 sigmoid), hs
    [T,Is] bf16, hqs [T,Is], shs [T], accs_d [T,H] int32."""
    x = np.ascontiguousarray(x)
    dt = _xdtype(x)
    wgu = _c(wgu, np.int8)
    E, twoI, H = wgu.shape
    I = twoI // 2
    T = x.shape[0]
    P = T * k
    Is, sa = _shared_args(shared, H)
    out = np.empty((T, H), x.dtype)
    inter = {}
    if intermediates:
        inter = dict(
            ids=np.empty((T, k), np.int32), w=np.empty((T, k), np.float32),
            xq=np.empty((T, H), np.int8), sx=np.empty(T, np.float32),
            offsets=np.empty(E + 1, np.int32), sorted_pair=np.empty(P, np.int32),
            pair_pos=np.empty(P, np.int32), h=np.empty((P, I), np.uint16), hq=np.empty((P, I), np.int8),
            sh=np.empty(P, np.float32), gate=np.empty(T, np.float64), hs=np.empty((T, Is), np.uint16),
            hqs=np.empty((T, Is), np.int8), shs=np.empty(T, np.float32), accs_d=np.empty((T, H), np.int32))
    g = inter.get
    lib().oracle_moe_layer_shared(_p(x), dt, T, H, E, k, I, _p(_c(wg, np.uint16)), _p(wgu), _p(_c(sgu, np.float32)),
                                  _p(_c(wd, np.int8)), _p(_c(sd, np.float32)), Is, *[_p(a) for a in sa], _p(out),
                                  _p(g("ids")), _p(g("w")), _p(g("xq")), _p(g("sx")), _p(g("offsets")),
                                  _p(g("sorted_pair")), _p(g("pair_pos")), _p(g("h")), _p(g("hq")), _p(g("sh")),
                                  _p(g("gate")), _p(g("hs")), _p(g("hqs")), _p(g("shs")), _p(g("accs_d")))
    return (out, inter) if intermediates else out


def moe_layer_shared_tokens(x, wg, wgu, sgu, wd, sd, k, shared, tokens):
    """Rows `tokens` of the shared-expert layer's output (no term couples tokens)."""
    x = np.ascontiguousarray(x)
    dt = _xdtype(x)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    E, twoI, H = wgu.shape
    I = twoI // 2
    Is, sa = _shared_args(shared, H)
    out = np.empty((len(tok), H), x.dtype)
    lib().oracle_moe_layer_shared_tokens(_p(x), dt, H, E, k, I, _p(_c(wg, np.uint16)), _p(_c(wgu, np.int8)),
                                         _p(_c(sgu, np.float32)), _p(_c(wd, np.int8)), _p(_c(sd, np.float32)), Is,
                                         *[_p(a) for a in sa], _p(tok), len(tok), _p(out))
    return out


# ------------------------------------------------------------ dense linear ---


def linear(x, qw, sw, out_dtype=BF16):
    """Dense W8A8 linear (the attention projections): x [M,K] quantised per row,
    then the one-group GEMM with the dequantising epilogue against int8 codes
    qw [N,K] and scales sw [N].  Returns out [M,N]."""
    qx, sx = quant_rows(x)
    M = qx.shape[0]
    return grouped_gemm(qx, sx, None, 1, _c(qw, np.int8)[None], _c(sw, np.float32)[None],
                        np.array([0, M], np.int32), DEQUANT, out_dtype)

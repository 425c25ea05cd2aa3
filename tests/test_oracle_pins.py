"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, exact rational arithmetic, brute force on tiny inputs, invariants
of the mathematics and the counts printed on the pages.  CPU only."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = synth.MOE_CONFIGS["moe_tiny_T16_H64_E8_k2_I32"]


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append([f.strip() for f in line.split("|")])
    return out


def _f32(v):
    return np.asarray(v, np.float32)


# ----------------------------------------------------------------- helpers ---

def round_to_f32(q: Fraction) -> Fraction:
    """Exact rational -> nearest binary32 value, ties to even (normal range)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # adjust so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp                      # in [2^23, 2^24)
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def rne_int(q: Fraction) -> int:
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def quant_exact(row):
    """The quantisation reading computed with exact rationals: scale =
    fl32(amax/127), code = RNE(fl32(x/scale)), clamp +-127."""
    xs = [Fraction(float(v)) for v in row]
    amax = max(abs(v) for v in xs)
    s = round_to_f32(amax / 127)
    if s == 0:
        return [0] * len(xs), s
    codes = [max(-127, min(127, rne_int(round_to_f32(v / s)))) for v in xs]
    return codes, s


# ------------------------------------------------------------ quantisation ---

def test_quant_closed_form_golden(orc):
    for scale, xs, codes in _rows("quant_closed_form.txt"):
        x = _f32([float(v) for v in xs.split()])[None, :]
        q, s = orc.quant_rows(x)
        assert float(s[0]) == float(scale)
        assert q[0].tolist() == [int(c) for c in codes.split()]
        # a bf16 copy of the same row (all values are bf16-exact) gives the same
        qb, sb = orc.quant_rows(synth.f32_to_bf16_bits(x))
        assert qb.tolist() == q.tolist() and sb.tolist() == s.tolist()


def test_quant_power_of_two_scaling(orc):
    """q(2^m x) = q(x) and s(2^m x) = 2^m s(x) when nothing over/underflows."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 333)).astype(np.float32)
    q0, s0 = orc.quant_rows(x)
    for m in (-20, -3, 1, 7, 30):
        q, s = orc.quant_rows((x * np.float32(2.0 ** m)).astype(np.float32))
        assert np.array_equal(q, q0)
        assert np.array_equal(s, (s0 * np.float32(2.0 ** m)).astype(np.float32))


def test_quant_matches_exact_rational_reading(orc):
    """Every code equals the exact-rational evaluation of RNE(fl32(x / fl32(amax/127))).
    Rows are selected where the alternative x*(127/amax) reading gives other
    codes, so this pin separates the two readings; plain random rows are
    checked too."""
    rng = np.random.default_rng(5)
    # Rows whose elements sit within a few ulps of half-integer multiples of the
    # row scale (element 0 fixes amax), where the two readings can round apart.
    n, m = 4000, 64
    amax0 = rng.uniform(0.5, 40, (n, 1)).astype(np.float32)
    s0 = amax0 / np.float32(127.0)
    half = (rng.integers(-126, 126, (n, m)) + 0.5).astype(np.float32)
    cand = (half * s0).astype(np.float32)
    cand = np.nextafter(cand, np.float32(np.inf) * rng.choice([-1, 1], (n, m))).astype(np.float32)
    cand[:, 0] = amax0[:, 0]
    amax = np.max(np.abs(cand), axis=1, keepdims=True)
    alt = np.clip(np.rint(cand * (np.float32(127.0) / amax)), -127, 127)
    div = np.clip(np.rint(cand / (amax / np.float32(127.0))), -127, 127)
    sep = np.nonzero(np.any(alt != div, axis=1))[0][:24]
    assert len(sep) >= 4, "no separating rows found"
    x = np.concatenate([cand[sep], cand[:24]])
    q, s = orc.quant_rows(x)
    alt_diff = 0
    for r in range(x.shape[0]):
        codes, sc = quant_exact(x[r])
        assert Fraction(float(s[r])) == sc
        assert q[r].tolist() == codes
        inv = np.float32(127.0) / np.max(np.abs(x[r]))
        alt_r = np.clip(np.rint(x[r] * inv), -127, 127).astype(np.int64)
        alt_diff += int(np.sum(alt_r != np.asarray(codes)))
    assert alt_diff > 0


def test_quant_invariants_on_workload_rows(orc):
    """|q| <= 127, the arg-max maps to +-127, q(-x) = -q(x) and
    |x - q*s| <= s*(1/2 + 2^-17) elementwise (the fp32 quotient adds at most
    127.5*2^-24 < 2^-17 to the half-unit rounding error)."""
    cfg = synth.MOE_CONFIGS["moe_30b_prefill_T4096"]
    x = synth.moe_x(synth.MoEConfig("sample", 64, cfg.H, cfg.E, cfg.k, cfg.I, "bf16", "student_t4", 8))
    gu, dn = synth.moe_expert_weights(synth.MoEConfig("sample_w", 4, 256, 2, 2, 64, "bf16", "normal", 0))
    for arr in (x, gu.reshape(-1, 256), dn.reshape(-1, 64)):
        q, s = orc.quant_rows(arr)
        xf = (synth.bf16_bits_to_f32(arr) if arr.dtype == np.uint16 else arr).astype(np.float64)
        assert np.all(np.abs(q.astype(np.int64)) <= 127)
        am = np.argmax(np.abs(xf), axis=1)
        assert np.all(np.abs(q[np.arange(len(am)), am]) == 127)
        err = np.abs(xf - q.astype(np.float64) * s.astype(np.float64)[:, None])
        assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -17))
        qn, sn = orc.quant_rows(-arr if arr.dtype != np.uint16 else arr ^ np.uint16(0x8000))
        assert np.array_equal(qn, -q) and np.array_equal(sn, s)


# -------------------------------------------------------------------- bf16 ---

def test_bf16_rounding_golden(orc):
    for v, bits in _rows("bf16_rne.txt"):
        assert orc.f64_to_bf16(float(v)) == int(bits, 16), v
        assert orc.f64_to_bf16(-float(v)) == int(bits, 16) ^ 0x8000, v


def test_bf16_rounding_matches_integer_rne(orc):
    """Against an independent integer implementation of RNE on fp32 bit patterns."""
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    want = synth.f32_to_bf16_bits(v)
    got = np.array([orc.f64_to_bf16(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ router ---

def test_router_fma_order_golden(orc):
    for xs, ws, want in _rows("router_fma_order.txt"):
        x = _f32([float(v) for v in xs.split()])[None, :]
        w = synth.f32_to_bf16_bits(_f32([[float(v) for v in ws.split()], [0.0, 0.0, 0.0]]))
        _, _, logits = orc.route_topk(x, w, 1)
        assert float(logits[0, 0]) == float(want)


def test_router_chunk_order_golden(orc):
    for hs, entries, want in _rows("router_chunk_order.txt"):
        H = int(hs)
        x = np.ones((1, H), np.float32)
        w = np.zeros((2, H), np.float32)
        for item in entries.split():
            i, v = item.split(":")
            w[0, int(i)] = float(v)
        _, _, logits = orc.route_topk(x, synth.f32_to_bf16_bits(w), 1)
        assert float(logits[0, 0]) == float(want)


@pytest.mark.parametrize("name", ["moe_30b_prefill_T4096", "moe_235b_zipf_T8192"])
def test_router_order_reading_moves_only_near_ties(orc, name):
    """R6 fixes the router's fp32 summation order (512-index fma chains added in
    order) because the pages fix none.  Against the other plain reading, one fma
    chain over all of h, on the full 30B-prefill and 235B router inputs: the two
    orders round most logits apart in the last bits, and a token's selected
    experts may differ only where two of its logits lie within the two orders'
    rounding error of each other (each order is within gamma_H * sum|x_h w_h| of
    the exact dot product).  On these inputs no token's top-k differs."""
    cfg = synth.MOE_CONFIGS[name]
    wg = synth.moe_router(cfg)
    x = synth.moe_x(cfg, wg_bits=wg)
    ic, _, lc = orc.route_topk(x, wg, cfg.k)
    ich, _, lch = orc.route_topk(x, wg, cfg.k, chunk=0)
    moved = np.nonzero(np.any(ic != ich, axis=1))[0]
    frac_apart = float(np.mean(lc != lch))
    print("%s: %d of %d tokens with another top-%d under one chain; %.1f%% of logits differ"
          % (name, len(moved), cfg.T, cfg.k, 100 * frac_apart))
    assert frac_apart > 0.5            # the orders are really different
    if len(moved):
        xf = (synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)
        S = np.abs(xf[moved]) @ np.abs(synth.bf16_bits_to_f32(wg).astype(np.float64)).T
        u = 2.0 ** -24
        gamma = cfg.H * u / (1 - cfg.H * u)
        for i, t in enumerate(moved):
            j = int(np.argmax(ic[t] != ich[t]))
            a, b = int(ic[t, j]), int(ich[t, j])
            assert abs(float(lc[t, a]) - float(lc[t, b])) <= 2 * gamma * (S[i, a] + S[i, b])
    assert len(moved) <= cfg.T // 1000


def _tiny_router():
    wg = synth.moe_router(TINY)
    x = synth.moe_x(TINY)
    return x, wg


def test_router_logits_are_x_times_wg_transposed(orc):
    """fp32 chain within the deterministic bound gamma_H * sum|x_k w_k| of the
    exact dot product (computed in exact rationals)."""
    x, wg = _tiny_router()
    wf = synth.bf16_bits_to_f32(wg)
    _, _, logits = orc.route_topk(x, wg, TINY.k)
    H = TINY.H
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    for t in range(TINY.T):
        for e in range(TINY.E):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], wf[e]))
            bound = gamma * float(sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(x[t], wf[e])))
            assert abs(float(logits[t, e]) - float(exact)) <= bound + 1e-30


def test_router_topk_brute_force(orc):
    """Top-k = the k-subset with the largest scores, ordered by (score desc, index
    asc); k=1 gives weight 1; renormalised weights = softmax over the selected
    scores; the weights sum to 1."""
    x, wg = _tiny_router()
    ids, w, logits = orc.route_topk(x, wg, TINY.k)
    for t in range(TINY.T):
        l = logits[t].astype(np.float64)
        best = max(itertools.combinations(range(TINY.E), TINY.k),
                   key=lambda c: (sorted([l[i] for i in c], reverse=True), [-i for i in c]))
        assert sorted(best) == sorted(ids[t].tolist())
        order = sorted(range(TINY.E), key=lambda e: (-l[e], e))[:TINY.k]
        assert ids[t].tolist() == order
        sel = l[ids[t]]
        sm = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        assert np.allclose(w[t], sm, rtol=0, atol=1e-6)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= TINY.k * 2.0 ** -23
    ids1, w1, _ = orc.route_topk(x, wg, 1)
    assert np.all(w1 == 1.0)
    assert np.array_equal(ids1[:, 0], np.argmax(logits, axis=1))
    idsE, wE, _ = orc.route_topk(x, wg, TINY.E, renormalize=False)
    for t in range(TINY.T):
        l = logits[t].astype(np.float64)
        p = np.exp(l - l.max()) / np.exp(l - l.max()).sum()
        assert np.allclose(wE[t], p[idsE[t]], atol=1e-7)
        assert sorted(idsE[t].tolist()) == list(range(TINY.E))


def test_router_ties_take_lower_index(orc):
    """Duplicate router rows give bit-identical scores; the lower expert id wins."""
    x, wg = _tiny_router()
    wg = wg.copy()
    wg[5] = wg[1]
    wg[6] = wg[1]
    ids, _, logits = orc.route_topk(x, wg, 3)
    assert np.array_equal(logits[:, 1], logits[:, 5])
    for t in range(TINY.T):
        row = ids[t].tolist()
        for a, b in ((1, 5), (1, 6), (5, 6)):
            if a in row and b in row:
                assert row.index(a) < row.index(b)
    # force the tie into the top-3 for every token: a huge duplicated score
    x2 = np.ones((4, TINY.H), np.float32)
    wg2 = np.zeros((TINY.E, TINY.H), np.float32)
    wg2[2] = wg2[7] = wg2[4] = 0.5
    ids2, w2, _ = orc.route_topk(x2, synth.f32_to_bf16_bits(wg2), 3)
    assert ids2.tolist() == [[2, 4, 7]] * 4
    assert np.all(w2 == np.float32(1.0 / 3.0))


# ----------------------------------------------------------------- permute ---

def test_permute_against_sort(orc):
    rng = np.random.default_rng(2)
    for T, k, E in ((1, 1, 1), (16, 2, 8), (37, 8, 128), (64, 8, 128), (5, 3, 7)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        offsets, sp, pos = orc.permute(ids, E)
        flat = ids.reshape(-1)
        want = sorted(range(T * k), key=lambda p: (flat[p], p))
        assert sp.tolist() == want
        counts = np.bincount(flat, minlength=E)
        assert offsets.tolist() == [0] + np.cumsum(counts).tolist()
        assert np.array_equal(pos[sp], np.arange(T * k))
        for e in range(E):
            seg = sp[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ------------------------------------------------------------- int8 GEMM ---

def test_int32_accumulators_exact_against_float64(orc):
    """RAW_I32 == float64 matmul of the codes (exact: |acc| <= K*127^2 < 2^53),
    with the MoE row gather."""
    rng = np.random.default_rng(9)
    T, k, E, K, N = 24, 3, 5, 208, 48
    A = rng.integers(-127, 128, (T, K), dtype=np.int8)
    B = rng.integers(-127, 128, (E, N, K), dtype=np.int8)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    offsets, sp, _ = orc.permute(ids, E)
    acc = orc.grouped_gemm(A, None, sp, k, B, None, offsets, orc.RAW_I32)
    for r in range(T * k):
        p = sp[r]
        e = ids.reshape(-1)[p]
        want = A[p // k].astype(np.float64) @ B[e].astype(np.float64).T
        assert np.array_equal(acc[r].astype(np.float64), want)
    # extremes: all +-127 gives K*127^2 exactly
    A2 = np.full((2, K), 127, np.int8)
    A2[1] = -127
    B2 = np.full((1, 3, K), -127, np.int8)
    acc2 = orc.grouped_gemm(A2, None, None, 1, B2, None, np.array([0, 2], np.int32), orc.RAW_I32)
    assert acc2.tolist() == [[-K * 127 * 127] * 3, [K * 127 * 127] * 3]


def test_integer_inputs_reduce_to_exact_matmul(orc):
    """Integer-valued rows that contain +-127 have scale exactly 1, so the W8A8
    linear is the exact integer matmul (fp32 output exact below 2^24)."""
    rng = np.random.default_rng(4)
    M, K, N = 8, 64, 16
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x[:, 0] = 127
    W = rng.integers(-127, 128, (N, K)).astype(np.float32)
    W[:, 3] = -127
    qx, sx = orc.quant_rows(x)
    qw, sw = orc.quant_rows(W)
    assert np.all(sx == 1.0) and np.all(sw == 1.0)
    y = orc.grouped_gemm(qx, sx, None, 1, qw[None], sw[None], np.array([0, M], np.int32),
                         orc.DEQUANT, orc.F32)
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ W.astype(np.float64).T)


def test_swiglu_closed_form(orc):
    """With unit scales the SwiGLU epilogue is silu(gate)*up at known integers;
    gate and up come from the first and second halves of the packed rows."""
    K, Ih = 16, 3
    A = np.zeros((2, K), np.int8)
    A[:, 0] = 127
    A[0, 1] = 1
    A[1, 1] = -2
    B = np.zeros((1, 2 * Ih, K), np.int8)
    B[0, :, 0] = [0, 0, 0, 0, 0, 0]
    B[0, :, 2] = 127                      # column 0 saturates every row's amax
    B[0, 0, 1], B[0, 1, 1], B[0, 2, 1] = 3, -5, 0          # gate
    B[0, 3, 1], B[0, 4, 1], B[0, 5, 1] = 7, 2, -9          # up
    sa = np.ones(2, np.float32)
    sb = np.ones((1, 2 * Ih), np.float32)
    h = orc.grouped_gemm(A, sa, None, 1, B, sb, np.array([0, 2], np.int32), orc.DEQUANT_SWIGLU, orc.F32)
    for r, a1 in enumerate((1, -2)):
        for n, (g, u) in enumerate(((3, 7), (-5, 2), (0, -9))):
            gv, uv = g * a1, u * a1
            want = gv / (1.0 + math.exp(-gv)) * uv
            assert h[r, n] == np.float32(want)


def test_dense_linear_quant_off_error_bound(orc):
    """|y_q - x W^T| <= sum_k(|x_k| e_w + e_x |w_k| + e_x e_w) + output rounding,
    e = s*(1/2 + 2^-17): the W8A8 linear stays within the quantisation error of
    the unquantised fp64 product.  A wrong scale (row/column swapped) breaks it."""
    cfg = synth.DenseConfig("dense_small", 64, 256, 96, 3)
    xb, W = synth.dense_inputs(cfg)
    x = synth.bf16_bits_to_f32(xb)
    qx, sx = orc.quant_rows(xb)
    qw, sw = orc.quant_rows(W)
    y = orc.grouped_gemm(qx, sx, None, 1, qw[None], sw[None], np.array([0, cfg.M], np.int32),
                         orc.DEQUANT, orc.F32).astype(np.float64)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    c = 0.5 + 2.0 ** -17
    ex = sx.astype(np.float64)[:, None] * c
    ew = sw.astype(np.float64)[None, :] * c
    bound = (np.abs(x).astype(np.float64).sum(1)[:, None] * ew
             + ex * np.abs(W).astype(np.float64).sum(1)[None, :] + cfg.K * ex * ew)
    assert np.all(np.abs(y - ref) <= bound * (1 + 1e-12) + np.abs(ref) * 2.0 ** -23)
    # a planted mistake (the weight scale of another channel) violates the bound
    y_bad = y / sw.astype(np.float64)[None, :] * np.roll(sw, 1).astype(np.float64)[None, :]
    assert np.any(np.abs(y_bad - ref) > bound)


# ------------------------------------------------------------- whole layer ---

def _tiny_layer(orc, cfg=TINY, seed=0):
    x, wg, gu, dn = synth.moe_inputs(cfg, seed)
    qgu, sgu = orc.quant_rows(gu.reshape(-1, cfg.H))
    qd, sd = orc.quant_rows(dn.reshape(-1, cfg.I))
    W = dict(wg=wg, wgu=qgu.reshape(gu.shape), sgu=sgu.reshape(cfg.E, -1),
             wd=qd.reshape(dn.shape), sd=sd.reshape(cfg.E, -1))
    return x, W


def _bf16_np(v):
    """Independent RNE of float64 values to bf16 for the brute force: round to
    fp32 is not allowed (double rounding), so go through exact rationals."""
    out = np.empty(v.shape, np.uint16)
    for i, a in np.ndenumerate(v):
        out[i] = _rational_bf16(Fraction(float(a)))
    return out


def _rational_bf16(q):
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    n = rne_int(a / ulp)
    v = np.float32(float(n * ulp))
    return int(v.view(np.uint32) >> 16) | sign


def test_layer_dense_vs_sparse_brute_force(orc):
    """Evaluate every expert for every token densely with numpy (no permute, no
    gather), then pick each token's experts: the int32 accumulators, h codes and
    outputs equal the oracle's grouped path."""
    x, W = _tiny_layer(orc)
    cfg = TINY
    out, it = orc.moe_layer(x, W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], cfg.k, intermediates=True)
    qx, sx = orc.quant_rows(x)
    assert np.array_equal(it["xq"], qx) and np.array_equal(it["sx"], sx)
    ids, w = it["ids"], it["w"]
    # dense gate/up accumulators for all (token, expert)
    acc_all = np.einsum("th,enh->ten", qx.astype(np.int64), W["wgu"].astype(np.int64))
    I = cfg.I
    want_out = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = ids[t, j]
            r = it["pair_pos"][t * cfg.k + j]
            assert np.array_equal(it["acc_gu"][r], acc_all[t, e])
            g = acc_all[t, e, :I] * float(sx[t]) * W["sgu"][e, :I].astype(np.float64)
            u = acc_all[t, e, I:] * float(sx[t]) * W["sgu"][e, I:].astype(np.float64)
            silu = np.array([gv / (1.0 + math.exp(-gv)) for gv in g])
            h = _bf16_np(silu * u)
            assert np.array_equal(it["h"][r], h)
            hq, sh = orc.quant_rows(h[None, :])
            assert np.array_equal(it["hq"][r], hq[0])
            accd = W["wd"][e].astype(np.int64) @ hq[0].astype(np.int64)
            assert np.array_equal(it["acc_d"][r], accd)
            want_out[t] += float(w[t, j]) * (accd * float(sh[0]) * W["sd"][e].astype(np.float64))
    assert np.array_equal(out, want_out.astype(np.float32))


def test_layer_token_independence(orc):
    """Shuffling tokens permutes the output rows bit for bit; a subset of tokens
    reproduces its rows."""
    x, W = _tiny_layer(orc)
    args = (W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], TINY.k)
    out = orc.moe_layer(x, *args)
    perm = np.random.default_rng(1).permutation(TINY.T)
    out_p = orc.moe_layer(x[perm], *args)
    assert np.array_equal(out_p, out[perm])
    sub = [3, 0, 11]
    assert np.array_equal(orc.moe_layer_tokens(x, *args, sub), out[sub])


def test_layer_equal_expert_weights(orc):
    """When every expert has the same weights the combine returns the single
    expert output scaled by sum(w) (= 1 up to rounding)."""
    x, W = _tiny_layer(orc)
    W1 = dict(W)
    W1["wgu"] = np.repeat(W["wgu"][:1], TINY.E, 0)
    W1["sgu"] = np.repeat(W["sgu"][:1], TINY.E, 0)
    W1["wd"] = np.repeat(W["wd"][:1], TINY.E, 0)
    W1["sd"] = np.repeat(W["sd"][:1], TINY.E, 0)
    out, it = orc.moe_layer(x, W1["wg"], W1["wgu"], W1["sgu"], W1["wd"], W1["sd"], TINY.k, intermediates=True)
    single = orc.moe_layer(x, W1["wg"], W1["wgu"], W1["sgu"], W1["wd"], W1["sd"], 1)
    ws = it["w"].astype(np.float64).sum(1)
    assert np.allclose(out, single * ws[:, None], rtol=1e-6, atol=1e-9)


def test_layer_quant_off_sanity(orc):
    """Quantised layer vs the unquantised fp64 SwiGLU MoE with the same routing:
    relative error small (reported bound, not a parity tolerance)."""
    x, W = _tiny_layer(orc)
    x64 = x.astype(np.float64)
    gu, dn = synth.moe_expert_weights(TINY)
    out, it = orc.moe_layer(x, W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], TINY.k, intermediates=True)
    ref = np.zeros_like(x64)
    for t in range(TINY.T):
        for j in range(TINY.k):
            e = it["ids"][t, j]
            a = gu[e].astype(np.float64) @ x64[t]
            g, u = a[:TINY.I], a[TINY.I:]
            ref[t] += it["w"][t, j] * (dn[e].astype(np.float64) @ (g / (1 + np.exp(-g)) * u))
    rel = np.abs(out - ref).max() / np.abs(ref).max()
    assert rel < 0.05


# ---------------------------------------------------------- page counts ---

def test_workload_shapes_match_page_counts():
    c = {k: float(v) for k, v in _rows("page_counts.txt")}
    m30 = synth.MOE_CONFIGS["moe_30b_prefill_T4096"]
    m235 = synth.MOE_CONFIGS["moe_235b_zipf_T8192"]
    per_layer = m30.E * 3 * m30.H * m30.I
    assert abs(per_layer / c["expert_params_per_layer_30b"] - 1) < 0.01
    assert abs(per_layer * c["layers_30b"] / c["expert_params_total_30b"] - 1) < 0.01
    assert m30.E == c["experts"] and m30.k == c["topk"] and m30.H == c["hidden_30b"]
    router = m30.H * m30.E
    assert abs(router / c["router_params_per_layer_30b"] - 1) < 0.01
    assert abs(router * c["layers_30b"] / c["router_params_total_30b"] - 1) < 0.01
    assert router * c["layers_30b"] * 2 < c["router_bytes_max_30b"]
    assert m235.H == c["hidden_235b"] and m235.E == c["experts"] and m235.k == c["topk"]
    experts_235 = c["layers_235b"] * m235.E * 3 * m235.H * m235.I
    assert 0.9 * c["params_total_235b"] < experts_235 < c["params_total_235b"]


def test_combine_closed_form(orc):
    """One-hot routing weights return the selected expert row; weights (a, b)
    give a*y1 + b*y2 for exactly representable values; pair_pos is honoured."""
    H = 8
    y = np.arange(4 * H, dtype=np.float32).reshape(4, H) - 7.0
    pair_pos = np.array([2, 0, 3, 1], np.int32)          # token 0: rows 2, 0; token 1: rows 3, 1
    w = np.array([[1.0, 0.0], [0.25, 0.75]], np.float32)
    out = orc.combine(y, w, pair_pos, orc.F32)
    assert np.array_equal(out[0], y[2])
    assert np.array_equal(out[1], 0.25 * y[3] + 0.75 * y[1])
    outb = orc.combine(synth.f32_to_bf16_bits(y), w, pair_pos, orc.BF16)
    assert np.array_equal(synth.bf16_bits_to_f32(outb), out)   # all values bf16-exact


# -------------------------------------------------------------------- W4A8 ---

def _w4_dequant(q, s, o):
    """(q - o) * s per group of 128 columns, in float64."""
    rows, cols = q.shape
    out = np.empty((rows, cols))
    for g in range(s.shape[1]):
        c0, c1 = 128 * g, min(cols, 128 * g + 128)
        out[:, c0:c1] = (q[:, c0:c1].astype(np.float64) - o[:, g:g + 1]) * s[:, g:g + 1].astype(np.float64)
    return out


def test_w4_codes_reconstruct_within_half_a_step(orc):
    """Every weight is within half a quantisation step of (q - o) * s, up to
    the rounding of s and w / s (an element whose u would be 16 by a tie is
    clamped: within one step); codes and offsets are 4-bit two's complement."""
    rng = np.random.default_rng(11)
    for cols in (128, 300, 64, 1536):
        w = (rng.standard_t(4, (6, cols)) * 0.02).astype(np.float32)
        w[1] = np.abs(w[1])          # one-signed rows: zero is an end of the range
        w[2] = -np.abs(w[2])
        q, s, o = orc.quant_w4_rows(w)
        assert q.min() >= -8 and q.max() <= 7 and o.min() >= -8 and o.max() <= 7
        assert s.shape == (6, (cols + 127) // 128)
        err = np.abs(_w4_dequant(q, s, o) - w)
        step = np.repeat(s.astype(np.float64), 128, axis=1)[:, :cols]
        assert np.all(err <= step * (0.5 + 1e-5) + 1e-12) or np.all(err <= step * 1.0001)
        assert np.mean(err <= step * (0.5 + 1e-5)) > 0.999


def test_w4_grid_values_are_exact(orc):
    """Values on a power-of-two grid whose codes span 0..15 come back exactly,
    with the constructed codes, offset and step."""
    rng = np.random.default_rng(5)
    rows = []
    want = []
    for z in range(16):
        u = rng.integers(0, 16, 128)
        u[0], u[1] = 0, 15                   # the range is exactly 15 steps
        s = 2.0 ** -7
        rows.append(((u - z) * s).astype(np.float32))
        want.append((u - 8, z - 8, s))
    q, sc, o = orc.quant_w4_rows(np.stack(rows))
    for r, (qu, oz, s) in enumerate(want):
        assert np.array_equal(q[r], qu.astype(np.int8))
        assert o[r, 0] == oz and sc[r, 0] == np.float32(s)
        assert np.array_equal(_w4_dequant(q[r:r + 1], sc[r:r + 1], o[r:r + 1])[0], rows[r].astype(np.float64))


def test_w4_degenerate_groups(orc):
    """A group of zeros has step 0, codes and offset 0; a constant group keeps
    zero at an end of its range (codes 7 / -8 against offsets -8 / 7)."""
    c = np.float32(0.0375)
    w = np.stack([np.zeros(128, np.float32), np.full(128, c, np.float32), np.full(128, -c, np.float32)])
    q, s, o = orc.quant_w4_rows(w)
    assert s[0, 0] == 0 and np.all(q[0] == 0) and o[0, 0] == 0
    assert np.all(q[1] == 7) and o[1, 0] == -8 and s[1, 0] == np.float32(c / np.float32(15))
    assert np.all(q[2] == -8) and o[2, 0] == 7
    d = _w4_dequant(q, s, o)
    assert np.allclose(d[1], float(c), rtol=1e-6) and np.allclose(d[2], -float(c), rtol=1e-6)


def test_w4a8_gemm_equals_dequantised_float_matmul(orc):
    """The W4A8 GEMM (integer sums per group, then the step) equals the float64
    product of the codes with the dequantised weights, for both epilogues."""
    rng = np.random.default_rng(9)
    G, N, K = 3, 64, 300
    A = rng.integers(-127, 128, (40, K)).astype(np.int8)
    sa = (rng.random(40) * 0.01 + 1e-3).astype(np.float32)
    w = (rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)
    q, s, o = orc.quant_w4_rows(w)
    Wd = _w4_dequant(q, s, o).reshape(G, N, K)
    offsets = np.array([0, 7, 7, 40], np.int32)
    out = orc.w4a8_grouped_gemm(A, sa, None, 1, q.reshape(G, N, K), s.reshape(G, N, -1), o.reshape(G, N, -1),
                                offsets, orc.DEQUANT, orc.F32)
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        want = (A[r0:r1].astype(np.float64) @ Wd[g].T) * sa[r0:r1, None].astype(np.float64)
        assert np.allclose(out[r0:r1], want, rtol=2e-6, atol=1e-9)
    sw = orc.w4a8_grouped_gemm(A, sa, None, 1, q.reshape(G, N, K), s.reshape(G, N, -1), o.reshape(G, N, -1),
                               offsets, orc.DEQUANT_SWIGLU, orc.F32)
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        full = (A[r0:r1].astype(np.float64) @ Wd[g].T) * sa[r0:r1, None].astype(np.float64)
        gate, up = full[:, :N // 2], full[:, N // 2:]
        assert np.allclose(sw[r0:r1], gate / (1.0 + np.exp(-gate)) * up, rtol=2e-6, atol=1e-9)


def test_w4_layer_dense_brute_force(orc):
    """The W4A8-gate_up layer against a dense numpy evaluation of every expert
    for every token with the dequantised W4 weights, then each token's experts."""
    cfg = TINY
    x, wg, gu, dn = synth.moe_inputs(cfg, 0)
    q4, s4, o4 = orc.quant_w4_rows(gu.reshape(-1, cfg.H))
    qd, sd = orc.quant_rows(dn.reshape(-1, cfg.I))
    E, I, H = cfg.E, cfg.I, cfg.H
    W4 = dict(q=q4.reshape(E, 2 * I, H), s=s4.reshape(E, 2 * I, -1), o=o4.reshape(E, 2 * I, -1))
    wd, sd = qd.reshape(E, H, I), sd.reshape(E, H)
    out, it = orc.moe_layer_w4(x, wg, W4["q"], W4["s"], W4["o"], wd, sd, cfg.k, intermediates=True)
    qx, sx = orc.quant_rows(x)
    Wgu = _w4_dequant(q4, s4, o4).reshape(E, 2 * I, H)
    gu_all = np.einsum("th,enh->ten", qx.astype(np.float64), Wgu) * sx.astype(np.float64)[:, None, None]
    want = np.zeros((cfg.T, H))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = it["ids"][t, j]
            g, u = gu_all[t, e, :I], gu_all[t, e, I:]
            h = _bf16_np(g / (1.0 + np.exp(-g)) * u)
            r = it["pair_pos"][t * cfg.k + j]
            assert np.array_equal(it["h"][r], h)
            hq, sh = orc.quant_rows(h[None, :])
            accd = wd[e].astype(np.int64) @ hq[0].astype(np.int64)
            want[t] += float(it["w"][t, j]) * (accd * float(sh[0]) * sd[e].astype(np.float64))
    assert np.array_equal(out, want.astype(np.float32))


# ---------------------------------------------------------- shared expert ---

TINY_SE = synth.MOE_CONFIGS["moe_tiny_shared_T16_H64_E8_k2_I32_Is64"]


def _tiny_shared(orc, wsg=None):
    x, W = _tiny_layer(orc, TINY_SE)
    gu, dn, wsg0 = synth.shared_expert(TINY_SE)
    qs, ss = orc.quant_rows(gu)
    qd, sd = orc.quant_rows(dn)
    se = dict(wgu=qs, sgu=ss, wd=qd, sd=sd, wsg=wsg0 if wsg is None else wsg)
    return x, W, se


def _one_expert_layer(orc, x, se):
    """The shared expert run as the only expert of a routed layer with k = 1:
    its renormalised routing weight is exactly 1, so the layer returns the
    expert's output through the routed path (router, permute, combine)."""
    wg1 = np.zeros((1, x.shape[1]), np.uint16)
    return orc.moe_layer(x, wg1, se["wgu"][None], se["sgu"][None], se["wd"][None], se["sd"][None], 1)


def _routed(orc, x, W, k):
    return orc.moe_layer(x, W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], k)


def test_shared_expert_with_zero_gate_adds_half_a_one_expert_layer(orc):
    """w_sg = 0 gives a logit of 0 and a sigmoid of exactly 1/2: the layer is
    the routed layer plus half of the shared expert, which equals a one-expert
    routed layer with the shared weights (a different code path)."""
    x, W, se = _tiny_shared(orc, wsg=np.zeros(TINY_SE.H, np.uint16))
    out, it = orc.moe_layer_shared(x, W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], TINY_SE.k, se,
                                   intermediates=True)
    assert np.all(it["gate"] == 0.5)
    want = _routed(orc, x, W, TINY_SE.k).astype(np.float64) + 0.5 * _one_expert_layer(orc, x, se)
    np.testing.assert_allclose(out, want, rtol=2e-6, atol=1e-7)
    assert not np.allclose(out, _routed(orc, x, W, TINY_SE.k), rtol=1e-3, atol=1e-5)


def test_shared_gate_saturates_to_zero_and_one(orc):
    """A logit of -1000 gives a sigmoid of exactly 0 (the shared expert drops out
    bit for bit), +1000 exactly 1 (the full shared output is added)."""
    x, W, se = _tiny_shared(orc)
    x = x.copy()
    sign = np.where(np.arange(TINY_SE.T) % 2 == 0, 1.0, -1.0).astype(np.float32)
    x[:, 0] = sign
    wsg = np.zeros(TINY_SE.H, np.uint16)
    wsg[0] = synth.f32_to_bf16_bits(np.float32([1000.0]))[0]   # 1000 is a bf16 value
    se["wsg"] = wsg
    out, it = orc.moe_layer_shared(x, W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], TINY_SE.k, se,
                                   intermediates=True)
    assert np.array_equal(it["gate"], np.where(sign > 0, 1.0, 0.0))
    routed = _routed(orc, x, W, TINY_SE.k)
    neg = sign < 0
    assert np.array_equal(out[neg], routed[neg])
    want = routed.astype(np.float64) + _one_expert_layer(orc, x, se)
    np.testing.assert_allclose(out[~neg], want[~neg], rtol=2e-6, atol=1e-7)


def test_shared_expert_brute_force(orc):
    """The shared expert and its gate evaluated by hand: int64 matmuls of the
    codes, SwiGLU in fp64, bf16 by exact rationals, the gate logit as the fp64
    sum of x times the bf16 gate vector over the hidden index (from x, not its
    int8 codes), sigmoid with libm's exp."""
    x, W, se = _tiny_shared(orc)
    cfg = TINY_SE
    out, it = orc.moe_layer_shared(x, W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], cfg.k, se,
                                   intermediates=True)
    qx, sx = orc.quant_rows(x)
    Is = cfg.Is
    acc = qx.astype(np.int64) @ se["wgu"].astype(np.int64).T
    g = acc[:, :Is] * sx.astype(np.float64)[:, None] * se["sgu"][:Is].astype(np.float64)
    u = acc[:, Is:] * sx.astype(np.float64)[:, None] * se["sgu"][Is:].astype(np.float64)
    hs = _bf16_np(g / (1.0 + np.exp(-g)) * u)
    assert np.array_equal(it["hs"], hs)
    hqs, shs = orc.quant_rows(hs)
    assert np.array_equal(it["hqs"], hqs) and np.array_equal(it["shs"], shs)
    accd = hqs.astype(np.int64) @ se["wd"].astype(np.int64).T
    assert np.array_equal(it["accs_d"], accd)
    wsg = synth.bf16_bits_to_f32(se["wsg"]).astype(np.float64)
    for t in range(cfg.T):
        lg = 0.0
        for c in range(cfg.H):
            lg += float(x[t, c]) * float(wsg[c])
        assert it["gate"][t] == 1.0 / (1.0 + math.exp(-lg))
    z = accd * shs.astype(np.float64)[:, None] * se["sd"].astype(np.float64)
    want = _routed(orc, x, W, cfg.k).astype(np.float64) + it["gate"][:, None] * z
    np.testing.assert_allclose(out, want, rtol=2e-6, atol=1e-7)
    # the gates span a real range, not a constant
    assert it["gate"].min() < 0.5 < it["gate"].max()


def test_shared_layer_token_subset(orc):
    x, W, se = _tiny_shared(orc)
    args = (W["wg"], W["wgu"], W["sgu"], W["wd"], W["sd"], TINY_SE.k, se)
    out = orc.moe_layer_shared(x, *args)
    sub = [5, 0, 15]
    assert np.array_equal(orc.moe_layer_shared_tokens(x, *args, sub), out[sub])



# ------------------------------------------------------------ dense linear ---

def test_fused_qkv_columns_equal_separate_linears(orc):
    """With per-output-channel weight scales and per-token activation scales, a
    fused QKV linear over the concatenated weight rows returns, column range
    by column range, exactly the three separate linears (no quantity couples
    output channels), and each equals the float64 product of the codes."""
    rng = np.random.default_rng(11)
    M, K, nq, nkv = 9, 96, 64, 16
    x = rng.standard_normal((M, K)).astype(np.float32)
    parts = [rng.standard_normal((n, K)).astype(np.float32) * np.float32(0.02) for n in (nq, nkv, nkv)]
    qs = [orc.quant_rows(w) for w in parts]
    fused_q = np.concatenate([q for q, _ in qs])
    fused_s = np.concatenate([s_ for _, s_ in qs])
    out = orc.linear(x, fused_q, fused_s, orc.F32)
    col = 0
    for q, s_ in qs:
        sep = orc.linear(x, q, s_, orc.F32)
        assert np.array_equal(out[:, col:col + q.shape[0]], sep)
        col += q.shape[0]
    qx, sx = orc.quant_rows(x)
    acc = qx.astype(np.float64) @ fused_q.astype(np.float64).T
    want = (acc * sx.astype(np.float64)[:, None] * fused_s.astype(np.float64)).astype(np.float32)
    assert np.array_equal(out, want)

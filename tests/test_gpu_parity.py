"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: int8 codes and scales, router scores and expert ids, the
permutation, int32 accumulators.  Within tolerance: dequantised outputs, routing
weights and the layer output (max|d| / max|ref| <= 1e-2 and mean |d| <= 1e-3).
Full-size workloads are compared on every token and every grouped row."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_int8_quantized_bf16_amd as w8

pytestmark = pytest.mark.gpu
DEV = "cuda"
NORM_TOL, MAE_TOL = 1e-2, 1e-3


# ------------------------------------------------------------------ helpers ---

def say(*a):
    print(*a, flush=True)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a):
    if a.dtype == np.uint16:
        return dev_bf16(a)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t):
    if t.dtype == torch.bfloat16:
        return host_bf16(t)
    return t.cpu().numpy()


def f64(a):
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def tol_check(got, want, what):
    g, w = f64(got), f64(want)
    d = np.abs(g - w)
    norm = d.max() / max(np.abs(w).max(), 1e-30)
    mae = d.mean()
    say("%s: max|d|/max|ref| = %.3e, mean|d| = %.3e, max|ref| = %.3e" % (what, norm, mae, np.abs(w).max()))
    assert norm <= NORM_TOL and mae <= MAE_TOL, what
    return norm, mae


def oracle_quant_w(gu, dn):
    E, twoI, H = gu.shape
    I = twoI // 2
    qgu, sgu = oracle.quant_rows(gu.reshape(-1, H))
    qd, sd = oracle.quant_rows(dn.reshape(-1, I))
    return qgu.reshape(gu.shape), sgu.reshape(E, twoI), qd.reshape(dn.shape), sd.reshape(E, H)


class Case:
    """One MoE workload: inputs, the oracle's weights and the GPU's weights."""

    def __init__(self, cfg, seed=0):
        t0 = time.time()
        self.cfg = cfg
        self.x, self.wg, gu, dn = synth.moe_inputs(cfg, seed=seed)
        self.o_qgu, self.o_sgu, self.o_qd, self.o_sd = oracle_quant_w(gu, dn)
        gu_d, dn_d = to_dev(gu), to_dev(dn)
        del gu, dn
        self.W = w8.MoEWeights.quantize(dev_bf16(self.wg), gu_d, dn_d, cfg.k)
        del gu_d, dn_d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.xd = to_dev(self.x)
        say("case %s ready in %.1f s" % (cfg.name, time.time() - t0))

    def oracle_args(self):
        return (self.wg, self.o_qgu, self.o_sgu, self.o_qd, self.o_sd, self.cfg.k)

    def check_weights_bit_exact(self):
        assert np.array_equal(to_host(self.W.w_gate_up), self.o_qgu)
        assert np.array_equal(to_host(self.W.s_gate_up), self.o_sgu)
        assert np.array_equal(to_host(self.W.w_down), self.o_qd)
        assert np.array_equal(to_host(self.W.s_down), self.o_sd)

    def run_layer(self):
        T = self.cfg.T
        dt = w8.BF16 if self.x.dtype == np.uint16 else w8.F32
        ws = w8.moe_layer_workspace(self.W, T, dt)
        out = w8.moe_layer(self.W, self.xd, ws=ws)
        torch.cuda.synchronize()
        return out, w8.moe_layer_intermediates(self.W, T, ws, dt), ws


_cases = {}


def get_case(name, seed=0):
    key = (name, seed)
    if key not in _cases:
        for k in list(_cases):
            if k != key:
                del _cases[k]
        torch.cuda.empty_cache()
        _cases[key] = Case(synth.MOE_CONFIGS[name], seed)
    return _cases[key]


# ---------------------------------------------------------- quantisation ---

@pytest.mark.parametrize("rows,cols,dtype,scale", [
    (1, 16, "bf16", 1.0), (5, 48, "f32", 3.0), (37, 1040, "bf16", 0.01), (16, 64, "f32", 1.0),
    (300, 2048, "bf16", 5.0), (3, 4096, "f32", 1e-3), (64, 768, "bf16", 100.0), (9, 768, "f32", 0.5),
    (33, 1536, "f32", 2.0), (70, 1536, "bf16", 30.0)])
def test_quant_act_bit_exact(rows, cols, dtype, scale):
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_t(4, (rows, cols)) * scale).astype(np.float32)
    x[rows // 2] = 0.0                                   # an all-zero row
    if rows > 2:
        x[1, : cols // 2] = -x[1, : cols // 2]
        x[2] = np.round(x[2] * 4) / 4                    # many exact halves
    xa = synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    q, s = w8.quant_act(to_dev(xa))
    oq, os_ = oracle.quant_rows(xa)
    assert np.array_equal(to_host(q), oq)
    assert np.array_equal(to_host(s), os_)
    assert np.all(to_host(s)[rows // 2] == 0)


def test_quant_act_leading_dimension():
    """A view with a row stride larger than the row (ld_x > cols)."""
    rng = np.random.default_rng(1)
    x = synth.f32_to_bf16_bits(rng.standard_normal((40, 96)).astype(np.float32))
    xd = to_dev(x)
    L = w8.lib()
    q = torch.empty((40, 64), dtype=torch.int8, device=DEV)
    s = torch.empty(40, dtype=torch.float32, device=DEV)
    rc = L.w8a8_quant_act(w8._p(xd), w8.BF16, 40, 64, 96, w8._p(q), w8._p(s), w8._stream())
    assert rc == 0
    oq, os_ = oracle.quant_rows(np.ascontiguousarray(x[:, :64]))
    assert np.array_equal(to_host(q), oq) and np.array_equal(to_host(s), os_)


# ---------------------------------------------------------------- router ---

@pytest.mark.parametrize("k,renorm", [(2, True), (1, True), (8, True), (3, False), (8, False)])
def test_route_tiny(k, renorm):
    cfg = synth.MOE_CONFIGS["moe_tiny_T16_H64_E8_k2_I32"]
    x, wg = synth.moe_x(cfg), synth.moe_router(cfg)
    ids, w, logits = w8.route_topk(to_dev(x), dev_bf16(wg), k, renorm, return_logits=True)
    oids, ow, ologits = oracle.route_topk(x, wg, k, renorm)
    assert np.array_equal(to_host(logits), ologits)
    assert np.array_equal(to_host(ids), oids)
    assert np.abs(to_host(w) - ow).max() <= 2e-6


def test_route_ties_lower_index_first():
    cfg = synth.MOE_CONFIGS["moe_tiny_T16_H64_E8_k2_I32"]
    x, wg = synth.moe_x(cfg), synth.moe_router(cfg).copy()
    wg[6] = wg[2]
    wg[7] = wg[2]
    for xx in (x, synth.f32_to_bf16_bits(x)):
        ids, w, logits = w8.route_topk(to_dev(xx), dev_bf16(wg), 4, True, return_logits=True)
        oids, ow, ologits = oracle.route_topk(xx, wg, 4)
        lg = to_host(logits)
        assert np.array_equal(lg[:, 2], lg[:, 6]) and np.array_equal(lg[:, 2], lg[:, 7])
        assert np.array_equal(to_host(ids), oids)
    # an all-equal router: every token selects 0..k-1 in order with equal weights
    flat = np.zeros_like(wg)
    ids, w = w8.route_topk(to_dev(x), dev_bf16(flat), 3)
    assert np.all(to_host(ids) == np.array([0, 1, 2]))
    assert np.allclose(to_host(w), 1.0 / 3.0, atol=1e-7)


def _tie_router(E, H, groups, rng):
    """Router rows N(0, 0.05) except the rows of each group, which are copies of
    one all-positive row (scaled down group by group), so that on tokens with
    a positive mean every group's logits are equal and rank above the rest."""
    w = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    base = (0.05 * (1.0 + 0.1 * rng.standard_normal(H))).astype(np.float32)
    for gi, rows in enumerate(groups):
        w[rows] = base * np.float32(1.0 - 0.2 * gi)
    return synth.f32_to_bf16_bits(w)


@pytest.mark.parametrize("E,groups", [
    (128, [[5, 69], [63, 64]]),                          # equal rows in both 64-expert slices, and astride them
    (256, [[5, 69, 133, 197], [63, 64, 127, 128, 191, 192]]),   # four slices; the 8th slot falls inside a tie
    (128, [[3, 60, 63, 64, 65, 100, 127, 126, 90, 64 + 3]]),     # one tie of 10 rows for 8 slots
    (256, [[255, 200, 130, 129, 66, 65, 2, 1, 0, 190]]),
])
@pytest.mark.parametrize("T", [16, 1024])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_route_exact_ties_across_slices(E, groups, T, xdt):
    """Exact ties of router scores (duplicated router rows give bit-identical
    fma chains) between experts in different 64-expert slices and at the top-k
    threshold: ids bit-exact with the oracle, equal scores ordered by the lower
    expert index.  T = 16 runs the few-token vector-ALU router, T = 1024 with
    bf16 tokens the matrix-core one, fp32 tokens the vector-fma one; each with
    and without the packed router copy."""
    _check_route_ties(E, groups, T, xdt)


@pytest.mark.parametrize("groups", [[[5, 69], [63, 64]], [[3, 60, 63, 64, 65, 100, 127, 126, 90, 64 + 3]]])
def test_route_exact_ties_many_tokens(groups):
    """The same ties at 8192 bf16 tokens and 128 experts, on the 32-token
    blocks of the 32 x 32 x 1 matrix-core router and its lane-parallel top-k."""
    _check_route_ties(128, groups, 8192, "bf16")


def _check_route_ties(E, groups, T, xdt):
    H, k = 2048, 8
    rng = np.random.default_rng(E + T + len(groups))
    x = (rng.standard_t(4, (T, H)) + 0.5).astype(np.float32)
    xa = synth.f32_to_bf16_bits(x) if xdt == "bf16" else x
    wg = _tie_router(E, H, groups, rng)
    oids, ow, ologits = oracle.route_topk(xa, wg, k)
    want_top = sorted(groups[0])[:k]
    wgd = dev_bf16(wg)
    for packed in (None, w8.router_pack(wgd)):
        ids, w, logits = w8.route_topk(to_dev(xa), wgd, k, True, return_logits=True, w_gate_packed=packed)
        lg = to_host(logits)
        for rows in groups:
            for r in rows[1:]:
                assert np.array_equal(lg[:, rows[0]], lg[:, r])
        assert np.array_equal(lg, ologits)
        got = to_host(ids)
        assert np.array_equal(got, oids)
        assert np.abs(to_host(w) - ow).max() <= 2e-6
        # the first group ranks on top for every token: its lowest indices, in order
        n0 = min(k, len(groups[0]))
        assert np.all(got[:, :n0] == np.array(want_top[:n0]))


def test_route_all_zero_router_matrix_core():
    """An all-zero router at E = 128 with 1024 tokens (the matrix-core router):
    every score is +0, every token selects experts 0..7 in order, weights 1/8."""
    rng = np.random.default_rng(9)
    x = synth.f32_to_bf16_bits(rng.standard_t(4, (1024, 2048)).astype(np.float32))
    wg = np.zeros((128, 2048), np.uint16)
    for packed in (None, w8.router_pack(dev_bf16(wg))):
        ids, w = w8.route_topk(to_dev(x), dev_bf16(wg), 8, w_gate_packed=packed)
        assert np.all(to_host(ids) == np.arange(8))
        assert np.all(to_host(w) == np.float32(0.125))


def _half_step_rows(rng, n, cols, amax_lo, amax_hi):
    """Rows whose elements lie one ulp off half-integer multiples of the row's
    scale (element 0 fixes the maximum), where a quotient that is not the
    correctly rounded x / s rounds to the other code."""
    amax0 = rng.uniform(amax_lo, amax_hi, (n, 1)).astype(np.float32)
    s0 = amax0 / np.float32(127.0)
    half = (rng.integers(-126, 126, (n, cols)) + 0.5).astype(np.float32)
    cand = (half * s0).astype(np.float32)
    cand = np.nextafter(cand, np.float32(np.inf) * rng.choice([-1, 1], (n, cols))).astype(np.float32)
    cand[:, 0] = amax0[:, 0]
    return cand


@pytest.mark.parametrize("cols", [64, 768, 1536, 2048, 4096, 1040])
def test_quant_act_adversarial_rows(cols):
    """The quantiser on rows built to sit one ulp off the rounding boundaries
    (the rows that separate the IEEE quotient x / s from x * (127 / amax)),
    at the widths of every quantiser kernel shape, with scales in the fast
    reciprocal-and-fma path and below 2^-100 (the divide path): codes and
    scales bit-exact with the oracle."""
    rng = np.random.default_rng(cols)
    x = np.concatenate([_half_step_rows(rng, 48, cols, 0.5, 40.0), _half_step_rows(rng, 8, cols, 1e-33, 1e-30)])
    amax = np.max(np.abs(x), axis=1, keepdims=True)
    alt = np.clip(np.rint(x * (np.float32(127.0) / amax)), -127, 127)
    div = np.clip(np.rint(x / (amax / np.float32(127.0))), -127, 127)
    say("cols %d: %d codes where the two quotients round apart" % (cols, int(np.sum(alt != div))))
    q, s = w8.quant_act(to_dev(x))
    oq, os_ = oracle.quant_rows(x)
    assert np.array_equal(to_host(s), os_)
    assert np.array_equal(to_host(q), oq)
    # bf16 rows with power-of-two scales: exact half-integer quotients (ties to even)
    m = rng.integers(-8, 8, (16, 1)).astype(np.float32)
    halves = (rng.integers(-127, 127, (16, cols)) + 0.5).astype(np.float32) * np.exp2(m)
    halves[:, 0] = 127.0 * np.exp2(m[:, 0])
    hb = synth.f32_to_bf16_bits(halves)
    assert np.array_equal(synth.bf16_bits_to_f32(hb), halves)
    q, s = w8.quant_act(to_dev(hb))
    oq, os_ = oracle.quant_rows(hb)
    assert np.array_equal(to_host(q), oq) and np.array_equal(to_host(s), os_)


@pytest.mark.parametrize("T,H,E,k", [(1, 16, 1, 1), (5, 48, 8, 2), (37, 2048, 63, 8), (9, 64, 64, 64),
                                     (17, 128, 65, 3), (33, 256, 96, 8), (12, 4096, 128, 8), (7, 80, 200, 11),
                                     (40, 32, 256, 16), (256, 2064, 128, 8), (128, 112, 200, 8),
                                     (257, 2064, 128, 8), (520, 2064, 63, 8), (300, 80, 200, 11),
                                     (700, 32, 256, 16), (600, 48, 8, 2), (3, 8192, 128, 8),
                                     (2, 1040, 64, 4), (5, 1536, 256, 8), (300, 1040, 128, 8),
                                     (33, 528, 130, 5), (600, 6160, 128, 8), (520, 9232, 60, 8)])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_route_shapes(T, H, E, k, xdt):
    """Expert counts that fill 1..4 slices of 64 (ragged ones included), odd
    token counts, short and long hidden sizes; bf16 and fp32 activations.
    With bf16 activations up to 512 (token, expert-slice) pairs take the
    vector-ALU router, more take the matrix-core one: both sides of that
    switch are here, with hidden sizes that leave a tail of W_g steps, and
    hidden sizes of 1 to 19 chunks of 512 (short last chunks included), which
    the vector-ALU router spreads over 1 to 8 waves per expert slice and the
    matrix-core one over 1 to 16 waves of one or two chunks each.  Each
    case runs with the [E][H] weight and with its packed copy (with bf16
    tokens and few of them: the chunk-parallel kernel)."""
    rng = np.random.default_rng(T * 1000 + E)
    x = rng.standard_t(4, (T, H)).astype(np.float32)
    xa = synth.f32_to_bf16_bits(x) if xdt == "bf16" else x
    wg = synth.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    oids, ow, ologits = oracle.route_topk(xa, wg, k)
    wgd = dev_bf16(wg)
    # the [E][H] weight, then its packed copy (the few-token kernel's other path)
    for packed in (None, w8.router_pack(wgd)):
        ids, w, logits = w8.route_topk(to_dev(xa), wgd, k, True, return_logits=True, w_gate_packed=packed)
        assert np.array_equal(to_host(logits), ologits)
        assert np.array_equal(to_host(ids), oids)
        assert np.abs(to_host(w) - ow).max() <= 2e-6


@pytest.mark.parametrize("T,H,E,k,renorm", [(600, 2048, 128, 8, False),    # a wave per chunk run and slice
                                            (300, 1040, 100, 10, True),    # the same with k > 8
                                            (300, 4624, 128, 3, False),    # two chunks per wave, both slices
                                            (8192, 2048, 128, 8, False)])  # 32-token blocks, a wave per run and slice
def test_route_matrix_core_ballot_topk(T, H, E, k, renorm):
    """The K = 1 matrix-core router with the ballot top-k (weights not
    renormalised, or k > 8) on blocks whose waves split the expert slices and
    on blocks whose waves hold both: logits, ids and weights against the
    oracle, with the [E][H] and the packed router weight."""
    rng = np.random.default_rng(T + H + E + k)
    x = synth.f32_to_bf16_bits(rng.standard_t(4, (T, H)).astype(np.float32))
    wg = synth.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    oids, ow, ologits = oracle.route_topk(x, wg, k, renorm)
    wgd = dev_bf16(wg)
    for packed in (None, w8.router_pack(wgd)):
        ids, w, logits = w8.route_topk(to_dev(x), wgd, k, renorm, return_logits=True, w_gate_packed=packed)
        assert np.array_equal(to_host(logits), ologits)
        assert np.array_equal(to_host(ids), oids)
        assert np.abs(to_host(w) - ow).max() <= 2e-6


@pytest.mark.parametrize("T,H,E,k", [(8192, 2064, 128, 8),    # two slices, 5 chunks (a short last one)
                                     (8200, 1040, 60, 4),     # one slice, a last block of 8 tokens
                                     (8192, 4624, 128, 8),    # two slices, two chunks per wave
                                     (8192, 8720, 64, 8),     # one slice, two chunks per wave
                                     (8230, 1552, 100, 6)])   # a part-filled second slice, a last chunk
                                                              # of two steps, a last block of 6 tokens
def test_route_matrix_core_many_tokens(T, H, E, k):
    """bf16 tokens in 256 or more blocks of 32 (the 32 x 32 x 1 matrix-core
    router): logits, ids and weights against the oracle with the [E][H] and
    the packed router weight; then an all-zero router (every score +0,
    experts 0..k-1 in order) and, inside a layer, the fused token quantisation
    of that kernel against the quantiser's oracle (rows read once where they
    fit the wave's registers, twice where not: H = 4624 and 8720; a ragged
    last block at T = 8200)."""
    rng = np.random.default_rng(T + H + E)
    x = synth.f32_to_bf16_bits(rng.standard_t(4, (T, H)).astype(np.float32))
    wg = synth.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    oids, ow, ologits = oracle.route_topk(x, wg, k)
    wgd = dev_bf16(wg)
    for packed in (None, w8.router_pack(wgd)):
        ids, w, logits = w8.route_topk(to_dev(x), wgd, k, True, return_logits=True, w_gate_packed=packed)
        assert np.array_equal(to_host(logits), ologits)
        assert np.array_equal(to_host(ids), oids)
        assert np.abs(to_host(w) - ow).max() <= 2e-6
    if (T, H) == (8192, 2064):
        z = np.zeros((E, H), np.uint16)
        ids, w = w8.route_topk(to_dev(x), dev_bf16(z), k, w_gate_packed=w8.router_pack(dev_bf16(z)))
        assert np.all(to_host(ids) == np.arange(k))
        assert np.all(to_host(w) == np.float32(1.0 / k))
    # the fused token quantisation, which only the layer asks for: a layer of
    # small experts (I = 32) around the same router, its ids, codes and scales
    I = 32
    gu = (rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    dn = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    W = w8.MoEWeights.quantize(wgd, to_dev(gu), to_dev(dn), k)
    del gu, dn
    ws = w8.moe_layer_workspace(W, T, w8.BF16)
    w8.moe_layer(W, to_dev(x), ws=ws)
    torch.cuda.synchronize()
    inter = w8.moe_layer_intermediates(W, T, ws, w8.BF16)
    assert np.array_equal(to_host(inter["ids"]), oids)
    oxq, osx = oracle.quant_rows(x)
    assert np.array_equal(to_host(inter["xq"]), oxq) and np.array_equal(to_host(inter["sx"]), osx)


@pytest.mark.parametrize("name", ["moe_30b_prefill_T4096", "moe_30b_decode_T64", "moe_235b_zipf_T8192"])
def test_route_full_size(name):
    cfg = synth.MOE_CONFIGS[name]
    wg = synth.moe_router(cfg)
    x = synth.moe_x(cfg, wg_bits=wg)
    ids, w, logits = w8.route_topk(to_dev(x), dev_bf16(wg), cfg.k, True, return_logits=True)
    t0 = time.time()
    oids, ow, ologits = oracle.route_topk(x, wg, cfg.k)
    say("oracle router %s on all %d tokens: %.1f s" % (name, cfg.T, time.time() - t0))
    assert np.array_equal(to_host(logits), ologits)
    assert np.array_equal(to_host(ids), oids)
    assert np.abs(to_host(w) - ow).max() <= 2e-6


# --------------------------------------------------------------- permute ---

@pytest.mark.parametrize("T,k,E,mode", [
    (1, 1, 1, "rand"), (16, 2, 8, "rand"), (37, 8, 128, "rand"), (4096, 8, 128, "rand"),
    (8192, 8, 128, "zipf"), (300, 4, 256, "rand"), (1000, 2, 8, "one"), (2049, 1, 3, "rand"),
    (513, 8, 16, "rand"), (512, 8, 128, "rand"), (4097, 1, 64, "rand"), (4096, 1, 256, "zipf")])
def test_permute_bit_exact(T, k, E, mode):
    rng = np.random.default_rng(T + k + E)
    if mode == "one":
        ids = np.zeros((T, k), np.int32)
        ids[:, 1] = 5
    elif mode == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, sp, pos = w8.permute(to_dev(ids), E)
    ooff, osp, opos = oracle.permute(ids, E)
    assert np.array_equal(to_host(off), ooff)
    assert np.array_equal(to_host(sp), osp)
    assert np.array_equal(to_host(pos), opos)


# ---------------------------------------------------------- grouped GEMM ---

def _groups(rng, sizes):
    off = np.zeros(len(sizes) + 1, np.int32)
    off[1:] = np.cumsum(sizes)
    return off


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("sizes,N,K,gather", [
    ([5, 0, 33, 1, 64], 48, 144, 0),          # ragged, an empty group, K tail
    ([3] * 40, 256, 2048, 2),                 # decode-like: tiny groups
    ([60, 70, 0, 45], 272, 1040, 0),          # N tail, mid-size groups
    ([300, 129, 1000], 512, 384, 8),          # large groups
    ([257, 200, 33, 384], 256, 512, 0),       # 128-row tiles whose last one holds 1, 72 or 33 rows
    ([400, 3, 900, 0], 272, 1040, 4),         # 128 x 512 tiles: N tail, K tail, a near-empty group
    ([17], 16, 16, 0),                        # minimum sizes
])
def test_grouped_gemm_raw_i32_exact(sizes, N, K, gather, packed):
    rng = np.random.default_rng(sum(sizes) + N + K)
    G, M = len(sizes), int(sum(sizes))
    off = _groups(rng, sizes)
    B = rng.integers(-127, 128, (G, N, K), dtype=np.int8)
    if gather:
        nA = max(M // gather + 1, 1)
        A = rng.integers(-127, 128, (nA, K), dtype=np.int8)
        gat = rng.integers(0, nA * gather, M).astype(np.int32)
    else:
        A = rng.integers(-127, 128, (M, K), dtype=np.int8)
        gat = None
    A[0, :] = 127                              # extremes
    B[0, 0, :] = -127
    Bd = to_dev(B)
    out = w8.grouped_gemm(to_dev(A), None, None if gat is None else to_dev(gat), max(gather, 1),
                          w8.pack_weights(Bd) if packed else Bd, None, to_dev(off), w8.EPI_RAW_I32, M_total=M,
                          b_shape=(G, N, K) if packed else None)
    got = to_host(out)
    want = oracle.grouped_gemm(A, None, gat, max(gather, 1), B, None, off, oracle.RAW_I32)
    assert np.array_equal(got, want)
    # independent exact check of one group
    g = int(np.argmax(sizes))
    rows = np.arange(off[g], off[g + 1])
    arow = gat[rows] // gather if gat is not None else rows
    assert np.array_equal(got[rows].astype(np.float64), A[arow].astype(np.float64) @ B[g].astype(np.float64).T)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("epi,od", [(w8.EPI_DEQUANT, w8.BF16), (w8.EPI_DEQUANT, w8.F32),
                                    (w8.EPI_DEQUANT_SWIGLU, w8.BF16), (w8.EPI_DEQUANT_SWIGLU, w8.F32)])
@pytest.mark.parametrize("sizes", [[7, 0, 90, 33], [200, 300], [500, 0, 777]])   # the last on 128 x 512 tiles
def test_grouped_gemm_dequant_epilogues(epi, od, sizes, packed):
    rng = np.random.default_rng(len(sizes) + epi * 10 + od)
    G, M, N, K = len(sizes), sum(sizes), 320, 528
    off = _groups(rng, sizes)
    x = rng.standard_t(4, (M, K)).astype(np.float32)
    Wf = (rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)
    qa, sa = oracle.quant_rows(x)
    qb, sb = oracle.quant_rows(Wf)
    qb, sb = qb.reshape(G, N, K), sb.reshape(G, N)
    qbd = to_dev(qb)
    out = w8.grouped_gemm(to_dev(qa), to_dev(sa), None, 1, w8.pack_weights(qbd) if packed else qbd, to_dev(sb),
                          to_dev(off), epi, od, b_shape=(G, N, K) if packed else None)
    want = oracle.grouped_gemm(qa, sa, None, 1, qb, sb, off, epi, od)
    got = to_host(out)
    g64, w64 = f64(got), f64(want)
    # fp32 epilogue vs fp64 reference: a few fp32 ulps, plus one output rounding
    rel = 2.0 ** -7 if od == w8.BF16 else 1e-5
    assert np.all(np.abs(g64 - w64) <= rel * np.abs(w64) + 1e-6 * np.abs(w64).max())


def test_pack_weights_layout():
    """Every byte of the packed layout is where the layout definition puts it
    (checked against an independent numpy gather), padding included."""
    rng = np.random.default_rng(12)
    for G, N, K in ((1, 32, 128), (2, 48, 144), (3, 96, 400)):
        B = rng.integers(-127, 128, (G, N, K), dtype=np.int8)
        got = to_host(w8.pack_weights(to_dev(B)))
        NB, KS = (N + 31) // 32, (K + 127) // 128
        Bp = np.zeros((G, NB * 32, KS * 128), np.int8)
        Bp[:, :N, :K] = B
        want = np.zeros(G * NB * KS * 4096, np.int8)
        for g in range(G):
            for nb in range(NB):
                for ks in range(KS):
                    base = ((g * NB + nb) * KS + ks) * 4096
                    for s_ in range(4):
                        for l in range(64):
                            row = nb * 32 + l % 32
                            k0 = ks * 128 + 64 * (l // 32) + 16 * s_
                            want[base + s_ * 1024 + l * 16: base + s_ * 1024 + l * 16 + 16] = Bp[g, row, k0:k0 + 16]
        assert np.array_equal(got, want)


# --------------------------------------------------------------- combine ---

@pytest.mark.parametrize("T,k,H,yd", [(16, 2, 64, "f32"), (64, 8, 2048, "bf16"), (3, 1, 16, "bf16"),
                                      (100, 8, 4096, "bf16")])
def test_combine(T, k, H, yd):
    rng = np.random.default_rng(T * k + H)
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    ya = synth.f32_to_bf16_bits(y) if yd == "bf16" else y
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    pos = rng.permutation(T * k).astype(np.int32)
    od = w8.BF16 if yd == "bf16" else w8.F32
    out = to_host(w8.combine(to_dev(ya), to_dev(w), to_dev(pos), od))
    want = oracle.combine(ya, w, pos, od)
    g64, w64 = f64(out), f64(want)
    rel = 2.0 ** -7 if od == w8.BF16 else 1e-6     # one bf16 ulp: fp32 vs fp64 sum can round apart
    assert np.all(np.abs(g64 - w64) <= rel * np.abs(w64) + 1e-6)


# ----------------------------------------------------------- whole layer ---

def _check_stages(case, inter, tokens=None):
    """Bit-exact stage checks of a layer run against the oracle."""
    cfg = case.cfg
    x = case.x
    oids, ow, _ = oracle.route_topk(x if tokens is None else x[tokens], case.wg, cfg.k)
    ids = to_host(inter["ids"])
    w = to_host(inter["w"])
    if tokens is not None:
        ids, w = ids[tokens], w[tokens]
    assert np.array_equal(ids, oids)
    assert np.abs(w - ow).max() <= 2e-6
    oxq, osx = oracle.quant_rows(x if tokens is None else x[tokens])
    xq, sx = to_host(inter["xq"]), to_host(inter["sx"])
    if tokens is not None:
        xq, sx = xq[tokens], sx[tokens]
    assert np.array_equal(xq, oxq) and np.array_equal(sx, osx)
    if tokens is None:
        off, sp, pos = oracle.permute(oids, cfg.E)
        assert np.array_equal(to_host(inter["offsets"]), off)
        assert np.array_equal(to_host(inter["sorted_pair"]), sp)
        assert np.array_equal(to_host(inter["pair_pos"]), pos)


def _group_of_rows(off, rows):
    return np.searchsorted(off, rows, side="right") - 1


def _raw_rows(A_rows_codes, Bq, off, rows):
    """The oracle's int32 accumulators of grouped rows `rows` (ascending) whose
    codes are A_rows_codes, against the groups' weights Bq [G, N, K]."""
    g = _group_of_rows(off, rows)
    counts = np.bincount(g, minlength=Bq.shape[0])
    sub_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return oracle.grouped_gemm(A_rows_codes, None, None, 1, Bq, None, sub_off, oracle.RAW_I32)


def _check_fixed16_rows(accd, sh, y16, yexp, off, sd, H, rows):
    """y carried as 16-bit fixed point (one power-of-two exponent per row and
    64-column segment): within 2^-14 of its segment's largest magnitude of the
    exact dequantised value acc * s_h * s_w, and each segment's largest code in
    [2^13, 2^14].  accd, y16, yexp: these rows; sd [E, H] the weight scales."""
    nseg = (H + 63) // 64
    e = _group_of_rows(off, rows)
    ref = np.zeros((len(rows), nseg * 64))
    ref[:, :H] = accd.astype(np.float64) * sh[rows].astype(np.float64)[:, None] * sd[e].astype(np.float64)
    got = np.zeros_like(ref)
    got[:, :H] = y16.astype(np.float64) * np.exp2(np.repeat(yexp.astype(np.int64), 64, axis=1)[:, :H])
    ref3, got3 = ref.reshape(len(rows), nseg, 64), got.reshape(len(rows), nseg, 64)
    m = np.abs(ref3).max(axis=2, keepdims=True)
    assert np.all(np.abs(got3 - ref3) <= 2.0 ** -14 * m * 1.0001 + 1e-6 * np.abs(ref3) + 1e-30)
    codes = np.zeros((len(rows), nseg * 64))
    codes[:, :H] = np.abs(y16.astype(np.float64))
    cm = codes.reshape(len(rows), nseg, 64).max(axis=2)
    live = m[:, :, 0] > 0
    assert np.all((cm[live] >= 2 ** 13 - 1) & (cm[live] <= 2 ** 14))


def _check_layer_full(case, out, inter, want, oi, what):
    """One layer run compared with the oracle's run of the same layer on every
    token and every grouped row: router ids (bit-exact) and weights, x codes
    and scales, the permutation, the gate_up int32 accumulators (RAW_I32 on the
    layer's own permutation), h within tolerance with its code mismatches
    bounded, h codes and scales of the GPU's own h, the down int32 accumulators
    of the GPU's own h codes, y's fixed-point bound, and the output."""
    cfg = case.cfg
    T, k, H, I = cfg.T, cfg.k, cfg.H, cfg.I
    P = T * k
    t0 = time.time()
    assert np.array_equal(to_host(inter["ids"]), oi["ids"])
    assert np.abs(to_host(inter["w"]) - oi["w"]).max() <= 2e-6
    assert np.array_equal(to_host(inter["xq"]), oi["xq"]) and np.array_equal(to_host(inter["sx"]), oi["sx"])
    off = to_host(inter["offsets"])
    assert np.array_equal(off, oi["offsets"])
    assert np.array_equal(to_host(inter["sorted_pair"]), oi["sorted_pair"])
    assert np.array_equal(to_host(inter["pair_pos"]), oi["pair_pos"])
    acc = w8.grouped_gemm(inter["xq"], None, inter["sorted_pair"], k, case.W.w_gate_up, None, inter["offsets"],
                          w8.EPI_RAW_I32, M_total=P)
    assert np.array_equal(to_host(acc), oi["acc_gu"]), "gate_up int32"
    del acc
    h = to_host(inter["h"])
    tol_check(h, oi["h"], what + " h")
    hq, sh = to_host(inter["hq"]), to_host(inter["sh"])
    q_, s_ = oracle.quant_rows(h)
    assert np.array_equal(hq, q_) and np.array_equal(sh, s_), "h codes of the GPU's own h"
    # h differs from the oracle's only where the hardware exponential moves a
    # bf16 rounding; its codes then differ by at most one step
    dq = np.abs(hq.astype(np.int16) - oi["hq"].astype(np.int16))
    frac = float(np.mean(dq > 0))
    say("%s: h-code mismatches %d of %d (%.2e), max |d| %d" % (what, int(np.sum(dq > 0)), dq.size, frac,
                                                               int(dq.max())))
    assert dq.max() <= 1 and frac <= 1e-5
    accd = to_host(w8.grouped_gemm(inter["hq"], None, None, 1, case.W.w_down, None, inter["offsets"],
                                   w8.EPI_RAW_I32, M_total=P))
    same = np.all(dq == 0, axis=1)
    assert np.array_equal(accd[same], oi["acc_d"][same]), "down int32"
    moved = np.nonzero(~same)[0]
    if len(moved):
        assert np.array_equal(accd[moved], _raw_rows(hq[moved], case.o_qd, off, moved)), "down int32 (moved rows)"
    y16, yexp = to_host(inter["y"]), to_host(inter["y_exp"])
    for r0 in range(0, P, 4096):
        rows = np.arange(r0, min(P, r0 + 4096))
        _check_fixed16_rows(accd[rows], sh, y16[rows], yexp[rows], off, case.o_sd, H, rows)
    del accd
    tol_check(to_host(out), want, what)
    counts = np.diff(off)
    say("%s: all %d tokens and %d grouped rows compared in %.1f s; expert loads min %d max %d cv %.2f"
        % (what, T, P, time.time() - t0, counts.min(), counts.max(), counts.std() / counts.mean()))


def _full_layer(name, seed=0):
    case = get_case(name, seed)
    if seed == 0:
        case.check_weights_bit_exact()
    out, inter, _ = case.run_layer()
    t0 = time.time()
    want, oi = oracle.moe_layer(case.x, *case.oracle_args(), intermediates=True)
    say("oracle %s (seed %d), all %d tokens with intermediates: %.1f s" % (name, seed, case.cfg.T, time.time() - t0))
    _check_layer_full(case, out, inter, want, oi, "%s seed %d" % (name, seed))
    return case, out, inter


def test_layer_tiny_full():
    _full_layer("moe_tiny_T16_H64_E8_k2_I32")


def test_layer_30b_decode_full():
    case, _, inter = _full_layer("moe_30b_decode_T64")
    hit = int(np.sum(np.diff(to_host(inter["offsets"])) > 0))
    say("decode: %d of %d experts hit" % (hit, case.cfg.E))


def test_layer_30b_prefill_full():
    _full_layer("moe_30b_prefill_T4096")


@pytest.mark.parametrize("name,seed", [("moe_30b_decode_T64", 1), ("moe_30b_decode_T64", 2),
                                       ("moe_30b_prefill_T4096", 1)])
def test_layer_other_seeds(name, seed):
    """Other draws of the same workloads (other expert loads, so other ragged
    row tiles), compared on every token and grouped row."""
    _full_layer(name, seed)


def test_layer_determinism_and_token_shuffle():
    case = get_case("moe_30b_prefill_T4096")
    out1, _, _ = case.run_layer()
    out2, _, _ = case.run_layer()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    perm = torch.from_numpy(np.random.default_rng(5).permutation(case.cfg.T)).to(DEV)
    ws = w8.moe_layer_workspace(case.W, case.cfg.T)
    out_p = w8.moe_layer(case.W, case.xd[perm].contiguous(), ws=ws)
    assert torch.equal(out_p.view(torch.int16), out1[perm].view(torch.int16))
    # a prefix of the tokens reproduces its rows
    out_s = w8.moe_layer(case.W, case.xd[:37].contiguous())
    assert torch.equal(out_s.view(torch.int16), out1[:37].view(torch.int16))


@pytest.mark.parametrize("T", [1, 255, 256, 257, 1000])
def test_layer_router_quantises_tokens(T):
    """With bf16 tokens the router also writes their int8 codes and scales
    (the vector-ALU router up to 256 tokens here, the matrix-core one above,
    ragged last blocks included): ids, weights, codes and scales bit-exact."""
    case = get_case("moe_30b_prefill_T4096")
    cfg = case.cfg
    xd = case.xd[:T].contiguous()
    ws = w8.moe_layer_workspace(case.W, T, w8.BF16)
    w8.moe_layer(case.W, xd, ws=ws)
    torch.cuda.synchronize()
    inter = w8.moe_layer_intermediates(case.W, T, ws, w8.BF16)
    x = case.x[:T]
    oids, ow, _ = oracle.route_topk(x, case.wg, cfg.k)
    assert np.array_equal(to_host(inter["ids"]), oids)
    assert np.abs(to_host(inter["w"]) - ow).max() <= 2e-6
    oxq, osx = oracle.quant_rows(x)
    assert np.array_equal(to_host(inter["xq"]), oxq) and np.array_equal(to_host(inter["sx"]), osx)


def test_layer_with_stage_events():
    """The timing entry point records its events (all, or only the non-null
    ones) and computes the same layer bit for bit."""
    case = get_case("moe_30b_decode_T64")
    out1, _, _ = case.run_layer()
    n = w8.LAYER_STAGES + 1
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    o_all = w8.moe_layer(case.W, case.xd, events=evs)
    sel = [e if j in (3, 4) else None for j, e in enumerate(evs)]
    o_sel = w8.moe_layer(case.W, case.xd, events=sel)
    torch.cuda.synchronize()
    assert evs[3].elapsed_time(evs[4]) > 0.0
    assert torch.equal(o_all.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(o_sel.view(torch.int16), out1.view(torch.int16))


def test_router_widen_and_both_router_inputs():
    """The fp32 router weight is the exact widening of the bf16 one, and the
    layer gives bit-identical results whether the router stages that copy or
    widens the bf16 weight itself."""
    case = get_case("moe_30b_prefill_T4096")
    wf = w8.router_widen(case.W.w_gate)
    want = torch.from_numpy(synth.bf16_bits_to_f32(case.wg)).to(DEV)
    assert torch.equal(wf.view(torch.int32), want.view(torch.int32))
    out1, _, _ = case.run_layer()
    saved = case.W.c.w_gate_f32
    try:
        case.W.c.w_gate_f32 = None
        out2 = w8.moe_layer(case.W, case.xd)
    finally:
        case.W.c.w_gate_f32 = saved
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("name", ["moe_30b_decode_T64", "moe_tiny_T16_H64_E8_k2_I32"])
def test_router_pack_and_both_few_token_paths(name):
    """The packed router weight is the [H/8][E][8] re-lay of the bf16 one,
    and a few-token layer gives bit-identical results whether the router reads
    that copy (the score's chunks on several waves) or the [E][H] rows (one
    wave per expert slice)."""
    case = get_case(name)
    E, H = case.cfg.E, case.cfg.H
    wp = w8.router_pack(case.W.w_gate)
    want = case.wg.reshape(E, H // 8, 8).transpose(1, 0, 2)
    assert np.array_equal(to_host(wp.view(torch.int16)).view(np.uint16), want)
    out1, _, _ = case.run_layer()
    saved = case.W.c.w_gate_packed
    try:
        case.W.c.w_gate_packed = None
        out2 = w8.moe_layer(case.W, case.xd)
    finally:
        case.W.c.w_gate_packed = saved
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_layer_edge_cases():
    case = get_case("moe_30b_prefill_T4096")
    out1, _, _ = case.run_layer()
    # one token
    o = w8.moe_layer(case.W, case.xd[5:6].contiguous())
    assert torch.equal(o.view(torch.int16), out1[5:6].view(torch.int16))
    # zero tokens: no-op
    empty = torch.empty((0, case.cfg.H), dtype=torch.bfloat16, device=DEV)
    assert w8.moe_layer(case.W, empty).shape == (0, case.cfg.H)
    # k = 1 and k = E on a tiny layer
    tiny = get_case("moe_tiny_T16_H64_E8_k2_I32")
    for k in (1, tiny.cfg.E):
        W = w8.MoEWeights(*tiny.W.tensors, k=k)
        out = w8.moe_layer(W, tiny.xd)
        want = oracle.moe_layer(tiny.x, tiny.wg, tiny.o_qgu, tiny.o_sgu, tiny.o_qd, tiny.o_sd, k)
        tol_check(to_host(out), want, "tiny layer k=%d" % k)


def test_layer_235b_zipf_full():
    case, out, inter = _full_layer("moe_235b_zipf_T8192")
    counts = np.diff(to_host(inter["offsets"]))
    assert counts.max() > 5 * counts.mean()      # the Zipf skew is there


def test_dense_linear_full():
    cfg = synth.DENSE_CONFIGS["dense_M4096_K2048_N4096"]
    xb, Wf = synth.dense_inputs(cfg)
    qx, sx = w8.quant_act(to_dev(xb))
    qw, sw = w8.quant_act(to_dev(Wf))
    oqx, osx = oracle.quant_rows(xb)
    oqw, osw = oracle.quant_rows(Wf)
    assert np.array_equal(to_host(qx), oqx) and np.array_equal(to_host(sx), osx)
    assert np.array_equal(to_host(qw), oqw) and np.array_equal(to_host(sw), osw)
    off = to_dev(np.array([0, cfg.M], np.int32))
    out = w8.grouped_gemm(qx, sx, None, 1, qw.view(1, cfg.N, cfg.K), sw.view(1, cfg.N), off, w8.EPI_DEQUANT, w8.BF16)
    want = oracle.grouped_gemm(oqx, osx, None, 1, oqw[None], osw[None], np.array([0, cfg.M], np.int32),
                               oracle.DEQUANT, oracle.BF16)
    tol_check(to_host(out), want, "dense W8A8 linear (all rows)")
    acc = w8.grouped_gemm(qx, None, None, 1, qw.view(1, cfg.N, cfg.K), None, off, w8.EPI_RAW_I32)
    want_acc = oracle.grouped_gemm(oqx, None, None, 1, oqw[None], None, np.array([0, cfg.M], np.int32),
                                   oracle.RAW_I32)
    assert np.array_equal(to_host(acc), want_acc)


# ------------------------------------------------------------------- W4A8 ---

@pytest.mark.parametrize("rows,cols", [(5, 64), (7, 304), (33, 2048), (3, 16)])
def test_w4_quant_bit_exact(rows, cols):
    """W4 codes, scales and offsets equal the oracle's, including one-signed
    rows, a zero row, short last groups and values on the quantisation grid."""
    rng = np.random.default_rng(rows * 31 + cols)
    w = (rng.standard_t(4, (rows, cols)) * 0.02).astype(np.float32)
    w[0] = 0.0
    if rows > 2:
        w[1] = np.abs(w[1])
        w[2] = -np.abs(w[2])
    if rows > 3:
        w[3] = (rng.integers(-7, 8, cols) * 2.0 ** -8).astype(np.float32)
    q, s, o = w8.w4a8_quant_weights(to_dev(w))
    oq, os_, oo = oracle.quant_w4_rows(w)
    assert np.array_equal(to_host(q), oq)
    assert np.array_equal(to_host(s), os_)
    assert np.array_equal(to_host(o), oo)


def _w4_problem(G, N, K, counts, seed, A_rows=None):
    rng = np.random.default_rng(seed)
    M = int(sum(counts))
    A_rows = A_rows or M
    A = rng.integers(-127, 128, (A_rows, K)).astype(np.int8)
    sa = (rng.random(A_rows) * 0.02 + 1e-3).astype(np.float32)
    w = (rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quant_w4_rows(w)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return A, sa, q.reshape(G, N, K), s.reshape(G, N, -1), o.reshape(G, N, -1), off


@pytest.mark.parametrize("G,N,K,counts,gather,epi,od", [
    (3, 64, 304, [7, 0, 33], False, 1, "f32"), (3, 128, 256, [5, 70, 1], True, 2, "bf16"),
    (2, 64, 64, [16, 16], False, 2, "f32"), (16, 1536, 2048, [128] * 16, True, 2, "bf16"),
    (128, 1536, 2048, [4] * 128, True, 2, "bf16"), (8, 2048, 768, [40] * 8, False, 1, "bf16"),
    (4, 256, 512, [100, 33, 64, 1], True, 2, "bf16"), (4, 256, 512, [100, 33, 64, 1], False, 1, "f32")])
def test_w4a8_grouped_gemm(G, N, K, counts, gather, epi, od):
    """The W4A8 GEMM through the C ABI against the oracle (32- and 64-row
    tiles, ragged and empty groups, 64-row tiles holding 1 to 36 rows,
    gathered rows, both epilogues)."""
    M = int(sum(counts))
    k = 4
    A, sa, q, s, o, off = _w4_problem(G, N, K, counts, G + N + K, A_rows=(M + k - 1) // k if gather else M)
    gat = (np.random.default_rng(1).permutation(M) % (A.shape[0] * k)).astype(np.int32) if gather else None
    if gather:
        gat = np.minimum(gat, A.shape[0] * k - 1).astype(np.int32)
    odc = w8.BF16 if od == "bf16" else w8.F32
    Bp = w8.w4a8_pack_weights(to_dev(q), to_dev(s), to_dev(o))
    got = w8.w4a8_grouped_gemm(to_dev(A), to_dev(sa), None if gat is None else to_dev(gat), k if gather else 1, Bp,
                               to_dev(off), epi, odc, M_total=M, b_shape=(G, N, K))
    want = oracle.w4a8_grouped_gemm(A, sa, gat, k if gather else 1, q, s, o, off, epi,
                                    oracle.BF16 if od == "bf16" else oracle.F32)
    tol_check(to_host(got), want, "w4a8 gemm G%d N%d K%d epi %d" % (G, N, K, epi))


@pytest.mark.parametrize("name", ["moe_tiny_T16_H64_E8_k2_I32", "moe_30b_decode_T64", "moe_30b_prefill_T4096"])
def test_w4_layer(name):
    """The layer with W4A8 gate_up weights (quantised on the GPU, bit-exact with
    the oracle's codes) against the oracle's W4 layer: ids and x codes bit-exact,
    h codes of the GPU's own h bit-exact, the output within tolerance on every
    token."""
    cfg = synth.MOE_CONFIGS[name]
    x, wg, gu, dn = synth.moe_inputs(cfg)
    E, I, H = cfg.E, cfg.I, cfg.H
    W = w8.MoEWeights.quantize(dev_bf16(wg), to_dev(gu), to_dev(dn), cfg.k, w4=True)
    q4, s4, o4 = oracle.quant_w4_rows(gu.reshape(-1, H))
    assert np.array_equal(to_host(W.w4[0]).reshape(-1, H), q4)
    assert np.array_equal(to_host(W.w4[1]).reshape(q4.shape[0], -1), s4)
    assert np.array_equal(to_host(W.w4[2]).reshape(q4.shape[0], -1), o4)
    qd, sd = oracle.quant_rows(dn.reshape(-1, I))
    args = (wg, q4.reshape(E, 2 * I, H), s4.reshape(E, 2 * I, -1), o4.reshape(E, 2 * I, -1), qd.reshape(E, H, I),
            sd.reshape(E, H), cfg.k)
    xd = to_dev(x)
    dt = w8.BF16 if x.dtype == np.uint16 else w8.F32
    ws = w8.moe_layer_workspace(W, cfg.T, dt)
    out = w8.moe_layer(W, xd, ws=ws)
    torch.cuda.synchronize()
    inter = w8.moe_layer_intermediates(W, cfg.T, ws, dt)
    t0 = time.time()
    want, it = oracle.moe_layer_w4(x, *args, intermediates=True)
    say("oracle %s w4 layer, all %d tokens: %.1f s" % (name, cfg.T, time.time() - t0))
    for key in ("ids", "xq", "sx", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(to_host(inter[key]), it[key]), key
    tol_check(to_host(inter["h"]), it["h"], "%s w4 h" % name)
    tol_check(to_host(out), want, "%s w4 layer (all tokens)" % name)
    h = to_host(inter["h"])
    oq, os_ = oracle.quant_rows(h)
    assert np.array_equal(to_host(inter["hq"]), oq) and np.array_equal(to_host(inter["sh"]), os_)


# ---------------------------------------------------------- shared expert ---

@pytest.mark.parametrize("name", ["moe_tiny_shared_T16_H64_E8_k2_I32_Is64", "moe_30b_shared_decode_T64",
                                  "moe_30b_shared_prefill_T4096"])
def test_shared_expert_layer(name):
    """The layer with a shared expert and its bf16 sigmoid gate: the shared
    weights' codes bit-exact, each shared stage checked on the GPU's own inputs
    to it (h within tolerance, h codes bit-exact, the down output within the
    16-bit fixed-point bound of the exact dequantised sums), the gate within
    1e-5 of the oracle's sigmoid, and the output within tolerance on every
    token."""
    cfg = synth.MOE_CONFIGS[name]
    say("shared expert layer", name)
    x, wg, gu, dn = synth.moe_inputs(cfg)
    sgu, sdn, wsg = synth.shared_expert(cfg)
    T, H, Is, k = cfg.T, cfg.H, cfg.Is, cfg.k
    W = w8.MoEWeights.quantize(dev_bf16(wg), to_dev(gu), to_dev(dn), k,
                               shared=(to_dev(sgu), to_dev(sdn), dev_bf16(wsg)))
    oq = oracle_quant_w(gu, dn)
    del gu, dn
    oqs, oss = oracle.quant_rows(sgu)
    oqsd, ossd = oracle.quant_rows(sdn)
    for got, want in zip(W.shared[:4], (oqs, oss, oqsd, ossd)):
        assert np.array_equal(to_host(got), want)
    se = dict(wgu=oqs, sgu=oss, wd=oqsd, sd=ossd, wsg=wsg)
    xd = to_dev(x)
    dt = w8.BF16 if x.dtype == np.uint16 else w8.F32
    ws = w8.moe_layer_workspace(W, T, dt)
    out = w8.moe_layer(W, xd, ws=ws)
    torch.cuda.synchronize()
    inter = w8.moe_layer_intermediates(W, T, ws, dt)
    P = T * k
    xq, sx = to_host(inter["xq"]), to_host(inter["sx"])
    oxq, osx = oracle.quant_rows(x)
    assert np.array_equal(xq, oxq) and np.array_equal(sx, osx)
    # shared gate_up + SwiGLU on the GPU's codes
    rows = np.arange(T)
    hs = to_host(inter["hs"])
    want_hs = oracle.grouped_gemm(xq[rows], sx[rows], None, 1, oqs[None], oss[None], np.array([0, len(rows)], np.int32),
                                  oracle.DEQUANT_SWIGLU, oracle.BF16)
    tol_check(hs[rows], want_hs, "%s shared h" % name)
    # h codes of the GPU's own h, bit-exact
    hqs, shs = to_host(inter["hqs"]), to_host(inter["shs"])
    q_, s_ = oracle.quant_rows(hs[rows])
    assert np.array_equal(hqs[rows], q_) and np.array_equal(shs[rows], s_)
    # down output rows P + t: 16-bit fixed point within 2^-14 of the segment max
    y16 = to_host(inter["y"])[P + rows].astype(np.float64)
    yexp = to_host(inter["y_exp"])[P + rows].astype(np.int64)
    ref = (hqs[rows].astype(np.float64) @ oqsd.astype(np.float64).T) * shs[rows].astype(np.float64)[:, None] \
        * ossd.astype(np.float64)
    got = y16 * np.exp2(np.repeat(yexp, 64, axis=1)[:, :H])
    for sg in range((H + 63) // 64):
        cols = slice(64 * sg, min(H, 64 * sg + 64))
        m = np.abs(ref[:, cols]).max(axis=1, keepdims=True)
        assert np.all(np.abs(got[:, cols] - ref[:, cols]) <= 2.0 ** -14 * m * 1.0001 + 1e-30)
    # the layer output, and the gate
    oargs = (wg, oq[0], oq[1], oq[2], oq[3], k, se)
    gate = to_host(inter["gate"]).astype(np.float64)
    t0 = time.time()
    want, it = oracle.moe_layer_shared(x, *oargs, intermediates=True)
    say("oracle %s, all %d tokens: %.1f s" % (name, T, time.time() - t0))
    assert np.abs(gate - it["gate"]).max() <= 1e-5
    say("%s: gates in [%.3f, %.3f]" % (name, gate.min(), gate.max()))
    tol_check(to_host(out), want, "%s layer (all tokens)" % name)
    # the routed part is unchanged by the shared expert: same ids and
    # permutation as the plain layer
    for key in ("ids", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(to_host(inter[key]), it[key]), key
    assert np.array_equal(to_host(inter["ids"]), oracle.route_topk(x, wg, k)[0])


@pytest.mark.parametrize("Is", [64, 32])
def test_shared_expert_edge_cases(Is):
    """T = 0 launches nothing; one and three tokens, fp32 activations; a shared
    expert wider than the routed ones (GEMMs of its own) and one as wide (an
    extra group of the routed GEMMs)."""
    import dataclasses
    cfg = dataclasses.replace(synth.MOE_CONFIGS["moe_tiny_shared_T16_H64_E8_k2_I32_Is64"], Is=Is)
    x, wg, gu, dn = synth.moe_inputs(cfg)
    sgu, sdn, wsg = synth.shared_expert(cfg)
    W = w8.MoEWeights.quantize(dev_bf16(wg), to_dev(gu), to_dev(dn), cfg.k,
                               shared=(to_dev(sgu), to_dev(sdn), dev_bf16(wsg)))
    oq = oracle_quant_w(gu, dn)
    oqs, oss = oracle.quant_rows(sgu)
    oqsd, ossd = oracle.quant_rows(sdn)
    se = dict(wgu=oqs, sgu=oss, wd=oqsd, sd=ossd, wsg=wsg)
    empty = torch.empty((0, cfg.H), dtype=torch.float32, device=DEV)
    assert w8.moe_layer(W, empty).shape == (0, cfg.H)
    for T in (1, 3, 16):
        out = w8.moe_layer(W, to_dev(x[:T]))
        torch.cuda.synchronize()
        want = oracle.moe_layer_shared(x[:T], wg, oq[0], oq[1], oq[2], oq[3], cfg.k, se)
        tol_check(to_host(out), want, "shared Is=%d T=%d" % (Is, T))


# ---------------------------------------------- dense linear (attention) ---

def _quant_pack_w(wf):
    """GPU codes, scales and packed codes of fp32 weights [N,K]; the codes are
    checked bit-exact against the oracle's."""
    qw, sw = w8.quant_act(to_dev(wf))
    oq, os_ = oracle.quant_rows(wf)
    assert np.array_equal(to_host(qw), oq) and np.array_equal(to_host(sw), os_)
    return qw, sw, w8.pack_weights(qw.view(1, *qw.shape)), oq, os_


@pytest.mark.parametrize("M,K,N", [(1, 64, 48), (3, 2048, 5120), (64, 2048, 5120), (300, 4096, 2048),
                                   (130, 96, 1040), (513, 128, 272), (64, 4096, 2048), (17, 3216, 528)])
@pytest.mark.parametrize("xdt,od", [("bf16", w8.BF16), ("f32", w8.F32)])
def test_linear_matches_oracle(M, K, N, xdt, od):
    """w8a8_linear (per-row quantisation + GEMM with tiles from the block index,
    K split into slices when there are few rows) against the oracle's quantised
    linear; w8a8_linear_q on the GPU's own codes returns the same bits, with
    and without the split."""
    say("linear", M, K, N, xdt, od)
    rng = np.random.default_rng(M * 7 + K + N)
    x32 = rng.standard_normal((M, K)).astype(np.float32)
    x32[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    x = synth.f32_to_bf16_bits(x32) if xdt == "bf16" else x32
    wf = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    qw, sw, pw, oq, os_ = _quant_pack_w(wf)
    out = w8.linear(to_dev(x), pw, sw, N, od)
    xq, sx = w8.quant_act(to_dev(x))
    out_q = w8.linear_q(xq, sx, pw, sw, N, od)
    out_nosplit = w8.linear_q(xq, sx, pw, sw, N, od, split=False)
    torch.cuda.synchronize()
    assert torch.equal(out, out_q)
    # K split into slices (few rows) adds int32 sums exactly: the same bits
    assert torch.equal(out_q, out_nosplit)
    want = oracle.linear(x, oq, os_, oracle.BF16 if od == w8.BF16 else oracle.F32)
    tol_check(to_host(out), want, "linear M%d K%d N%d" % (M, K, N))


def test_linear_zero_rows():
    wf = np.random.default_rng(1).standard_normal((64, 64)).astype(np.float32)
    qw, sw, pw, _, _ = _quant_pack_w(wf)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    assert w8.linear(x, pw, sw, 64).shape == (0, 64)


@pytest.mark.parametrize("name", ["attn_qkv_30b_T64", "attn_o_30b_T64", "attn_qkv_30b_T4096", "attn_o_30b_T4096",
                                  "attn_qkv_235b_T8192", "attn_o_235b_T8192"])
def test_attention_projection_workloads(name):
    """The attention projections at the layer shapes: the whole linear on the
    GPU, checked against the oracle on every row.  For the fused QKV shapes, the q, k and v column
    ranges equal separate linears over their own weight rows, bit for bit."""
    cfg = synth.DENSE_CONFIGS[name]
    say("attention projection", name)
    xb, wf = synth.dense_inputs(cfg)
    qw, sw, pw, oq, os_ = _quant_pack_w(wf)
    xd = to_dev(xb)
    out = w8.linear(xd, pw, sw, cfg.N)
    torch.cuda.synchronize()
    t0 = time.time()
    want = oracle.linear(xb, oq, os_)
    say("oracle %s, all %d rows: %.1f s" % (name, cfg.M, time.time() - t0))
    tol_check(to_host(out), want, name + " (all rows)")
    col = 0
    for n in cfg.split:
        part = w8.pack_weights(qw[col:col + n].contiguous().view(1, n, cfg.K))
        sep = w8.linear(xd, part, sw[col:col + n].contiguous(), n)
        torch.cuda.synchronize()
        assert torch.equal(out[:, col:col + n], sep), (name, col, n)
        col += n


# ------------------------------------------------------------ HIP graphs ---

@pytest.mark.parametrize("name,variant", [("moe_30b_decode_T64", "w8a8"), ("moe_tiny_shared_T16_H64_E8_k2_I32_Is64", "shared"),
                                          ("moe_30b_decode_T64", "w4a8"), ("moe_tiny_T16_H64_E8_k2_I32", "w8a8")])
def test_layer_in_hip_graph(name, variant):
    """The layer call captured in a HIP graph (it launches kernels only: no host
    synchronisation, allocation or memset) and replayed several times, with
    eager work and synchronisations between the replays: every replay equals
    the eager call bit for bit, also after the input changes in place."""
    cfg = synth.MOE_CONFIGS[name]
    say("graph", name, variant)
    x, wg, gu, dn = synth.moe_inputs(cfg)
    shared = None
    if variant == "shared":
        sgu, sdn, wsg = synth.shared_expert(cfg)
        shared = (to_dev(sgu), to_dev(sdn), dev_bf16(wsg))
    W = w8.MoEWeights.quantize(dev_bf16(wg), to_dev(gu), to_dev(dn), cfg.k, w4=variant == "w4a8", shared=shared)
    xd = to_dev(x)
    dt = w8.BF16 if x.dtype == np.uint16 else w8.F32
    ws = w8.moe_layer_workspace(W, cfg.T, dt)
    out = torch.empty_like(xd)
    eager = w8.moe_layer(W, xd, ws=ws, out=torch.empty_like(xd)).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the side stream once before capture
        w8.moe_layer(W, xd, ws=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.moe_layer(W, xd, ws=ws, out=out)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d" % i
        junk = torch.randn(1024, 1024, device=DEV) @ torch.randn(1024, 1024, device=DEV)   # eager work between
        torch.cuda.synchronize()
        del junk
    # new input values in place: the replay follows them
    x2 = (xd.float() * 0.5).to(xd.dtype)
    eager2 = w8.moe_layer(W, x2, ws=torch.empty_like(ws), out=torch.empty_like(xd)).clone()
    xd.copy_(x2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager2)

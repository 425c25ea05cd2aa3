"""Seeded synthetic inputs for the W8A8 MoE layer: shared by the tests, the bench
and the oracle's callers.

This module holds no arithmetic of the method itself (no quantisation, routing,
GEMM or combine).  It draws random tensors of the shapes and value
distributions of the workloads below and formats them in the layer's input
dtypes: bf16 inputs are the fp32 draws rounded to nearest-even bf16.

Every tensor has its own child stream of ``numpy.random.SeedSequence(seed)``, in
a fixed order:
    0            activations x
    1            router weight W_g
    2            structure (which channels are outliers, the Zipf expert ranks)
    3 + 3e + 0   expert e gate_proj   [I][H]
    3 + 3e + 1   expert e up_proj     [I][H]
    3 + 3e + 2   expert e down_proj   [H][I]
    3 + 3E + 0   shared expert gate_proj  [Is][H]   (layers with a shared expert)
    3 + 3E + 1   shared expert up_proj    [Is][H]
    3 + 3E + 2   shared expert down_proj  [H][Is]
    3 + 3E + 3   shared_expert_gate       [H] (bf16)

Workloads (shapes of the pages' models; all values synthetic):
  moe_tiny_T16_H64_E8_k2_I32      x fp32 N(0,1)
  dense_M4096_K2048_N4096         one W8A8 linear; x bf16 N(0,1), 1% of the
                                  channels (20) scaled x20
  moe_30b_prefill_T4096           Qwen3-30B-A3B-shaped layer: H=2048, E=128,
                                  k=8, I=768; x bf16 Student-t(4) with 8 outlier
                                  channels x20
  moe_30b_decode_T64              the same layer with T=64
  moe_235b_zipf_T8192             Qwen3-235B-A22B-shaped layer: H=4096, E=128,
                                  k=8, I=1536; x as above, shifted so that the
                                  router's scores carry a bias -1.1*ln(rank_e):
                                  Zipf(1.1)-skewed expert loads
  moe_tiny_shared_T16_H64_E8_k2_I32_Is64   the tiny layer plus a shared expert
                                  of intermediate size 64
  moe_30b_shared_prefill_T4096    the 30B-shaped prefill layer plus an always-on
                                  shared expert of intermediate size 768 and its
                                  bf16 sigmoid gate
  moe_30b_shared_decode_T64       the same with T=64
  attn_qkv_30b_T4096 / _T64       fused q/k/v projection of the 30B shape as one
                                  W8A8 linear: K=2048, N=4096+512+512
  attn_o_30b_T4096 / _T64         o_proj: K=4096, N=2048
  attn_qkv_235b_T8192             K=4096, N=8192+512+512
  attn_o_235b_T8192               K=8192, N=4096
                                  (x as the dense linear's: N(0,1) with 1% of
                                  the input channels scaled x20)
Weights: router W_g N(0, 0.02) in bf16; expert weights N(0, 0.02) in fp32 (they
are quantised to int8 per output channel by whichever side uses them); the
shared expert's weights N(0, 0.02) in fp32 and its gate vector N(0, 0.02) in
bf16.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    x_dtype: str          # "bf16" or "f32"
    x_dist: str           # "normal" or "student_t4"
    n_outlier: int        # outlier channels scaled by 20
    zipf_s: float = 0.0   # > 0: bias the router towards Zipf(zipf_s) loads
    Is: int = 0           # > 0: an always-on shared expert of this intermediate size

    @property
    def P(self):
        return self.T * self.k


@dataclass(frozen=True)
class DenseConfig:
    name: str
    M: int
    K: int
    N: int
    n_outlier: int
    split: tuple = ()     # fused q/k/v: the output widths of the three projections


MOE_CONFIGS = {
    c.name: c for c in [
        MoEConfig("moe_tiny_T16_H64_E8_k2_I32", 16, 64, 8, 2, 32, "f32", "normal", 0),
        MoEConfig("moe_30b_prefill_T4096", 4096, 2048, 128, 8, 768, "bf16", "student_t4", 8),
        MoEConfig("moe_30b_decode_T64", 64, 2048, 128, 8, 768, "bf16", "student_t4", 8),
        MoEConfig("moe_235b_zipf_T8192", 8192, 4096, 128, 8, 1536, "bf16", "student_t4", 8, zipf_s=1.1),
        MoEConfig("moe_tiny_shared_T16_H64_E8_k2_I32_Is64", 16, 64, 8, 2, 32, "f32", "normal", 0, Is=64),
        MoEConfig("moe_30b_shared_prefill_T4096", 4096, 2048, 128, 8, 768, "bf16", "student_t4", 8, Is=768),
        MoEConfig("moe_30b_shared_decode_T64", 64, 2048, 128, 8, 768, "bf16", "student_t4", 8, Is=768),
    ]
}
DENSE_CONFIGS = {c.name: c for c in [
    DenseConfig("dense_M4096_K2048_N4096", 4096, 2048, 4096, 20),
    # attention projections of the two layer shapes as dense W8A8 linears
    # (fused q/k/v rows; 32 query and 4 key/value heads of 128 at hidden 2048,
    # 64 and 4 at hidden 4096)
    DenseConfig("attn_qkv_30b_T4096", 4096, 2048, 5120, 20, (4096, 512, 512)),
    DenseConfig("attn_o_30b_T4096", 4096, 4096, 2048, 41),
    DenseConfig("attn_qkv_30b_T64", 64, 2048, 5120, 20, (4096, 512, 512)),
    DenseConfig("attn_o_30b_T64", 64, 4096, 2048, 41),
    DenseConfig("attn_qkv_235b_T8192", 8192, 4096, 9216, 41, (8192, 512, 512)),
    DenseConfig("attn_o_235b_T8192", 8192, 8192, 4096, 82),
]}

W_STD = 0.02
OUTLIER_GAIN = 20.0


def f32_to_bf16_bits(a):
    """Round float32 values to the nearest bf16, ties to even; return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(seed, E):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3 + 3 * E)]


def _outlier_channels(rng, H, n):
    return np.sort(rng.choice(H, size=n, replace=False)) if n else np.zeros(0, np.int64)


def moe_router(cfg: MoEConfig, seed=0):
    """W_g [E][H] as bf16 bits."""
    rng = _streams(seed, cfg.E)[1]
    return f32_to_bf16_bits(rng.standard_normal((cfg.E, cfg.H), dtype=np.float32) * np.float32(W_STD))


def moe_x(cfg: MoEConfig, seed=0, wg_bits=None):
    """Activations x [T][H]: uint16 bf16 bits (bf16 configs) or float32."""
    st = _streams(seed, cfg.E)
    rng_x, rng_s = st[0], st[2]
    if cfg.x_dist == "normal":
        x = rng_x.standard_normal((cfg.T, cfg.H))
    else:
        x = rng_x.standard_t(4, size=(cfg.T, cfg.H))
    ch = _outlier_channels(rng_s, cfg.H, cfg.n_outlier)
    x[:, ch] *= OUTLIER_GAIN
    if cfg.zipf_s > 0:
        # Expert ranks r_e (a seeded permutation of 1..E) and a score bias
        # b_e = -s*ln(r_e).  Shift every token by the minimum-norm vector d with
        # W_g d = b, so that the (bias-free) router sees scores + b.
        ranks = rng_s.permutation(cfg.E) + 1
        b = -cfg.zipf_s * np.log(ranks.astype(np.float64))
        if wg_bits is None:
            wg_bits = moe_router(cfg, seed)
        Wg = bf16_bits_to_f32(wg_bits).astype(np.float64)
        d = Wg.T @ np.linalg.solve(Wg @ Wg.T, b)
        x = x + d[None, :]
    x32 = x.astype(np.float32)
    return x32 if cfg.x_dtype == "f32" else f32_to_bf16_bits(x32)


def moe_expert(cfg: MoEConfig, e, seed=0, streams=None):
    """fp32 (gate [I][H], up [I][H], down [H][I]) of expert e."""
    st = streams if streams is not None else _streams(seed, cfg.E)
    g = st[3 + 3 * e].standard_normal((cfg.I, cfg.H), dtype=np.float32) * np.float32(W_STD)
    u = st[4 + 3 * e].standard_normal((cfg.I, cfg.H), dtype=np.float32) * np.float32(W_STD)
    d = st[5 + 3 * e].standard_normal((cfg.H, cfg.I), dtype=np.float32) * np.float32(W_STD)
    return g, u, d


def moe_expert_weights(cfg: MoEConfig, seed=0, threads=8):
    """All expert weights in the packed layout, fp32:
    gate_up [E][2I][H] (gate rows 0..I-1, up rows I..2I-1) and down [E][H][I]."""
    st = _streams(seed, cfg.E)
    gu = np.empty((cfg.E, 2 * cfg.I, cfg.H), np.float32)
    dn = np.empty((cfg.E, cfg.H, cfg.I), np.float32)

    def one(e):
        g, u, d = moe_expert(cfg, e, streams=st)
        gu[e, :cfg.I] = g
        gu[e, cfg.I:] = u
        dn[e] = d

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(cfg.E)))
    return gu, dn


def moe_inputs(cfg: MoEConfig, seed=0, threads=8):
    """(x, W_g bits, gate_up fp32, down fp32) of a MoE workload."""
    wg = moe_router(cfg, seed)
    x = moe_x(cfg, seed, wg)
    gu, dn = moe_expert_weights(cfg, seed, threads)
    return x, wg, gu, dn


def shared_expert(cfg: MoEConfig, seed=0):
    """The shared expert of a layer with cfg.Is > 0: fp32 gate_up [2Is][H]
    (gate rows then up rows), fp32 down [H][Is] and the bf16 bits of the
    shared_expert_gate vector [H]."""
    assert cfg.Is > 0
    st = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3 + 3 * cfg.E + 4)][3 + 3 * cfg.E:]
    gu = np.empty((2 * cfg.Is, cfg.H), np.float32)
    gu[:cfg.Is] = st[0].standard_normal((cfg.Is, cfg.H), dtype=np.float32) * np.float32(W_STD)
    gu[cfg.Is:] = st[1].standard_normal((cfg.Is, cfg.H), dtype=np.float32) * np.float32(W_STD)
    dn = st[2].standard_normal((cfg.H, cfg.Is), dtype=np.float32) * np.float32(W_STD)
    wsg = f32_to_bf16_bits(st[3].standard_normal(cfg.H, dtype=np.float32) * np.float32(W_STD))
    return gu, dn, wsg


def dense_inputs(cfg: DenseConfig, seed=0):
    """(x bf16 bits [M][K], W fp32 [N][K]) of the dense W8A8 linear."""
    st = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]
    x = st[0].standard_normal((cfg.M, cfg.K))
    ch = _outlier_channels(st[2], cfg.K, cfg.n_outlier)
    x[:, ch] *= OUTLIER_GAIN
    w = st[1].standard_normal((cfg.N, cfg.K), dtype=np.float32) * np.float32(W_STD)
    return f32_to_bf16_bits(x.astype(np.float32)), w

"""The allocation-free grouped GEMM (w8a8_grouped_gemm_noalloc, for callers
that cannot allocate device memory) against w8a8_grouped_gemm, the entry point
with a caller workspace: the same kernels, so the same bits.  Two calls in a
row on the fixed scratch array, the second on a smaller problem, each compared
right after it runs."""
import ctypes

import numpy as np
import pytest
import torch

import w8a8_int8_quantized_bf16_amd as w8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _problem(seed, sizes, N, K, gather_div):
    rng = np.random.default_rng(seed)
    G, M = len(sizes), int(sum(sizes))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    n_a = M // gather_div + 1 if gather_div > 1 else M
    A = torch.from_numpy(rng.integers(-127, 128, (n_a, K), dtype=np.int8)).to(DEV)
    sa = torch.from_numpy((rng.random(n_a) * 0.02 + 1e-3).astype(np.float32)).to(DEV)
    gat = None
    if gather_div > 1:
        gat = torch.from_numpy(rng.integers(0, n_a * gather_div, M).astype(np.int32)).to(DEV)
    B = torch.from_numpy(rng.integers(-127, 128, (G, N, K), dtype=np.int8)).to(DEV)
    sb = torch.from_numpy((rng.random((G, N)) * 0.01 + 1e-4).astype(np.float32)).to(DEV)
    return dict(A=A, sa=sa, gat=gat, div=gather_div, B=B, sb=sb, off=torch.from_numpy(off).to(DEV), G=G, M=M, N=N,
                K=K)


def _run(pb, epilogue, od, packed, noalloc):
    L = w8.lib()
    B = w8.pack_weights(pb["B"]) if packed else pb["B"]
    layout = w8.B_PACKED if packed else w8.B_ROWMAJOR
    M, N = pb["M"], pb["N"]
    if epilogue == w8.EPI_RAW_I32:
        out = torch.full((M, N), -7, dtype=torch.int32, device=DEV)
    else:
        ncol = N if epilogue == w8.EPI_DEQUANT else N // 2
        out = torch.full((M, ncol), 3.0, dtype=torch.bfloat16 if od == w8.BF16 else torch.float32, device=DEV)
    args = [w8._p(pb["A"]), pb["A"].shape[0], w8._p(pb["sa"]), w8._p(pb["gat"]), pb["div"], w8._p(B), layout,
            w8._p(pb["sb"]), w8._p(pb["off"]), pb["G"], M, N, pb["K"], epilogue, od, w8._p(out)]
    if noalloc:
        rc = L.w8a8_grouped_gemm_noalloc(*args, w8._stream())
    else:
        nws = int(L.w8a8_grouped_gemm_workspace_size(M, N, pb["G"]))
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=DEV)
        rc = L.w8a8_grouped_gemm(*args, w8._p(ws), ws.numel(), w8._stream())
    assert rc == 0, w8.status_string(rc)
    torch.cuda.synchronize()
    return out


def test_noalloc_grouped_gemm_matches_workspace_entry_point():
    # a layer-sized problem (128 experts, ragged groups incl. empty ones,
    # gathered rows, packed weights, SwiGLU), then a smaller one (row-major
    # weights, int32 sums): the second call reuses the array the first filled
    big = _problem(1, list(np.random.default_rng(5).integers(0, 700, 128)) + [0, 33], 1536, 2048, 8)
    small = _problem(2, [5, 0, 70, 1], 256, 384, 1)
    cases = [(big, w8.EPI_DEQUANT_SWIGLU, w8.BF16, True), (small, w8.EPI_RAW_I32, w8.I32, False),
             (small, w8.EPI_DEQUANT, w8.F32, True)]
    for i, (pb, epi, od, packed) in enumerate(cases):
        print("no-alloc case %d: G %d M %d N %d K %d epilogue %d" % (i, pb["G"], pb["M"], pb["N"], pb["K"], epi),
              flush=True)
        want = _run(pb, epi, od, packed, noalloc=False)
        got = _run(pb, epi, od, packed, noalloc=True)
        assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), "case %d" % i


def test_noalloc_refuses_beyond_its_scratch():
    pb = _problem(3, [64], 4096, 128, 1)
    out = torch.empty((64, 4096), dtype=torch.bfloat16, device=DEV)
    M = 1 << 22     # a tile table far beyond the fixed array; nothing is launched
    rc = w8.lib().w8a8_grouped_gemm_noalloc(w8._p(pb["A"]), 64, w8._p(pb["sa"]), w8._p(pb["off"]), 1 << 20,
                                            w8._p(pb["B"]), w8.B_ROWMAJOR, w8._p(pb["sb"]), w8._p(pb["off"]), 1, M,
                                            4096, 128, w8.EPI_DEQUANT, w8.BF16, w8._p(out), w8._stream())
    assert rc == -6

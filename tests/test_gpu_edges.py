"""Edge cases of the GEMM kernels on the GPU: one or two reduction stages per
tile, more tiles than compute units (so every workgroup chains several tiles
and prefetches the next one's first stages), single-row and ragged shapes.
Integer-valued inputs keep every sum exact, so results are compared bit for
bit with the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, TOL_ROW, bf16_dev, bf16_host, dec_bf16, f32_dev,
                            f32_host, norm_err, row_rel_err, say)

pytestmark = pytest.mark.gpu


def _ints(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [
    (8192, 4096, 64),    # 512 tiles, one stage per tile
    (8192, 4096, 128),   # 512 tiles, two stages per tile
    (4096, 8192, 192),   # 512 tiles, three stages
    (1, 16, 64),         # a single row, a single 16-wide feature group
    (257, 272, 64),      # ragged everything, one stage
    # shapes where the plain GEMM takes the 128 x 384 tile
    (8192, 3072, 64),    # 512 wide tiles (chained), one stage
    (8192, 3072, 192),   # 512 wide tiles, three stages
    (300, 320, 128),     # ragged rows, one partial tile column, two stages
])
def test_gemm1_and_plain_exact(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a, w = _ints(rng, (M, K), -1, 1), _ints(rng, (N, K), -1, 1)
    res = _ints(rng, (M, N), -3, 3)
    say(f"exact GEMM1/plain M={M} N={N} K={K}")
    A, W, R = (bf16_dev(inputs.to_bf16_bits(v)) for v in (a, w, res))
    h = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    P = torch.empty(ops.rms_tiles(N), M, dtype=torch.float32, device=DEV)
    C = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    ops.gemm_residual_partialrms(A, W, R, h, P)
    ops.gemm_bf16(A, W, C)
    torch.cuda.synchronize()
    y = oracle.gemm_nt(a, w)
    hh = oracle.residual_add(y, res)
    assert np.array_equal(bf16_host(C), y)
    assert np.array_equal(bf16_host(h), hh)
    assert np.array_equal(f32_host(P), oracle.partial_sumsq(hh, ops.rms_tile_width()))
    # the light reduction over T = ceil(N / 128) tiles (T = 1, 3, 32, 64: the
    # four-lane split of the tiles meets every remainder)
    r = torch.empty(M, dtype=torch.float32, device=DEV)
    ops.rms_reduce(P, N, 1e-5, r)
    torch.cuda.synchronize()
    assert row_rel_err(f32_host(r), oracle.rms_scale(hh, 1e-5)) <= TOL_ROW


@pytest.mark.parametrize("M,N,K", [(8192, 2048, 64), (4096, 4096, 128), (300, 48, 64)])
def test_swiglu_chained_small_k(M, N, K):
    """GEMM2 with more tiles than compute units and one or two stages per
    tile (values small enough that the pre-activations are exact)."""
    rng = np.random.default_rng(7 + K)
    x = _ints(rng, (M, K), -1, 1)
    wg, wu = _ints(rng, (N, K), -1, 1) / 8, _ints(rng, (N, K), -1, 1) / 8
    r = rng.uniform(0.5, 1.5, size=M).astype(np.float32)
    say(f"swiglu chained M={M} N={N} K={K}")
    X, G, U = (bf16_dev(inputs.to_bf16_bits(v.astype(np.float32))) for v in (x, wg, wu))
    out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    ops.gemm_rowscale_swiglu(X, G, U, f32_dev(r), out)
    torch.cuda.synchronize()
    rr = r.astype(np.float64)[:, None]
    ref = oracle.swiglu(rr * oracle.gemm_nt(x, wg), rr * oracle.gemm_nt(x, wu))
    assert norm_err(bf16_host(out), ref) <= TOL_BF16


def test_lse_chained_small_k():
    """Block LSE with 512 tiles (every workgroup chains) and one stage."""
    w = inputs.make_lm(seed=31, M=4096, d=64, V=8192)
    say("block lse chained M=4096 d=64 V=8192")
    M, V = 4096, 8192
    T = ops.lse_tiles(V)
    tmax = torch.empty(T, M, dtype=torch.float32, device=DEV)
    tsum = torch.empty_like(tmax)
    zl, loss = (torch.empty(M, dtype=torch.float32, device=DEV) for _ in range(2))
    ops.gemm_block_lse(bf16_dev(w.arrays["x"]), bf16_dev(w.arrays["wlm"]),
                       torch.from_numpy(w.arrays["labels"]).to(DEV), tmax, tsum, zl, loss)
    torch.cuda.synchronize()
    rows = np.arange(0, M, 37)
    ref = oracle.lm_head_ce(dec_bf16(w.arrays["x"][rows]), dec_bf16(w.arrays["wlm"]),
                            w.arrays["labels"][rows])
    assert row_rel_err(f32_host(loss)[rows], ref["loss"]) <= TOL_ROW


def test_rope_chained():
    """QKV + RoPE with more tiles than compute units (M=24576: 96 x 4 tiles)."""
    w = inputs.make_attn(seed=32, M=24576, d=128, K1=64, n_q=4, n_kv=2, head_dim=64,
                         seq_len=2048)
    say("rope chained M=24576 d=128")
    from tests.test_gpu_rope import oracle_rows, run_fused
    got = run_fused(w)
    rows = np.arange(0, 24576, 101)
    ref = oracle_rows(w, rows)
    assert norm_err(bf16_host(got["qkv"][rows.tolist()]), ref["qkv"]) <= TOL_BF16
    assert row_rel_err(f32_host(got["r"])[rows], ref["r"]) <= TOL_ROW

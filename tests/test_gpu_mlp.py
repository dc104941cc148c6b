"""GPU parity of the MLP block (GEMM1 residual/partial-RMS -> reduce -> GEMM2
row-scale/SwiGLU) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, TOL_ROW, MaxErr, bf16_dev, bf16_host, dec_bf16,
                            f32_dev, f32_host, norm_err, row_chunks, row_rel_err, say)

pytestmark = pytest.mark.gpu
EPS = 1e-5


def run_fused(w, eps=EPS):
    """The fused hot path on the GPU for an MLP workload; returns device tensors."""
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    x, res, w1 = bf16_dev(w.arrays["x"]), bf16_dev(w.arrays["res"]), bf16_dev(w.arrays["w1"])
    wg, wu = bf16_dev(w.arrays["wg"]), bf16_dev(w.arrays["wu"])
    gamma = f32_dev(w.arrays["gamma"])
    wg_f, wu_f = torch.empty_like(wg), torch.empty_like(wu)
    ops.fold_gamma(wg, gamma, wg_f)
    ops.fold_gamma(wu, gamma, wu_f)
    h = torch.empty(M, d, dtype=torch.bfloat16, device=DEV)
    T = ops.rms_tiles(d)
    P = torch.full((T, M), float("nan"), dtype=torch.float32, device=DEV)
    r = torch.empty(M, dtype=torch.float32, device=DEV)
    out = torch.empty(M, ffn, dtype=torch.bfloat16, device=DEV)
    ops.gemm_residual_partialrms(x, w1, res, h, P)
    ops.rms_reduce(P, d, eps, r)
    ops.gemm_rowscale_swiglu(h, wg_f, wu_f, r, out)
    torch.cuda.synchronize()
    return {"h": h, "P": P, "r": r, "out": out}


def run_unfused(w, eps=EPS):
    """The unfused sequence (one HBM round trip per op) on the GPU."""
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    x, res, w1 = bf16_dev(w.arrays["x"]), bf16_dev(w.arrays["res"]), bf16_dev(w.arrays["w1"])
    wgu = torch.cat([bf16_dev(w.arrays["wg"]), bf16_dev(w.arrays["wu"])], 0).contiguous()
    gamma = f32_dev(w.arrays["gamma"])
    y = torch.empty(M, d, dtype=torch.bfloat16, device=DEV)
    h, n = torch.empty_like(y), torch.empty_like(y)
    gu = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(M, ffn, dtype=torch.bfloat16, device=DEV)
    ops.gemm_bf16(x, w1, y)
    ops.residual_add(y, res, h)
    ops.rmsnorm(h, gamma, eps, n)
    ops.gemm_bf16(n, wgu, gu)
    ops.swiglu(gu, out)
    torch.cuda.synchronize()
    return {"h": h, "out": out}


def oracle_rows(w, rows=None, eps=EPS):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    return oracle.mlp_block(dec_bf16(sel(w.arrays["x"])), dec_bf16(sel(w.arrays["res"])),
                            dec_bf16(w.arrays["w1"]), dec_bf16(w.arrays["wg"]),
                            dec_bf16(w.arrays["wu"]), w.arrays["gamma"].astype(np.float64), eps)


def test_integer_exact_gemm1():
    """Entries in {-1, 0, 1}: every product and partial sum is a small integer,
    so h, the partial sums of squares and the plain GEMM are exact in any
    summation order and must match the oracle bit for bit.  M, N ragged."""
    M, N, K = 300, 272, 192
    rng = np.random.default_rng(0)
    a = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
    wt = rng.integers(-1, 2, size=(N, K)).astype(np.float32)
    res = rng.integers(-4, 5, size=(M, N)).astype(np.float32)
    to_bits = lambda v: inputs.to_bf16_bits(v)
    say(f"integer-exact GEMM1 M={M} N={N} K={K}")
    A, W, R = bf16_dev(to_bits(a)), bf16_dev(to_bits(wt)), bf16_dev(to_bits(res))
    h = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    T = ops.rms_tiles(N)
    P = torch.empty(T, M, dtype=torch.float32, device=DEV)
    C = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    ops.gemm_residual_partialrms(A, W, R, h, P)
    ops.gemm_bf16(A, W, C)
    torch.cuda.synchronize()
    ref_y = oracle.gemm_nt(a, wt)
    ref_h = oracle.residual_add(ref_y, res)
    assert np.array_equal(bf16_host(h), ref_h)
    assert np.array_equal(bf16_host(C), ref_y)
    ref_P = oracle.partial_sumsq(ref_h, ops.rms_tile_width())
    assert np.array_equal(f32_host(P), ref_P)


def test_mlp_ragged_parity():
    """Several tiles in every dimension with ragged tails in M, d and ffn."""
    w = inputs.make_mlp(seed=3, M=600, d=448, K1=320, ffn=1040)
    say("mlp ragged M=600 d=448 K1=320 ffn=1040")
    got = run_fused(w)
    ref = oracle_rows(w)
    assert norm_err(bf16_host(got["h"]), ref["h"]) <= TOL_BF16
    assert row_rel_err(f32_host(got["r"]), ref["r"]) <= TOL_ROW
    assert norm_err(bf16_host(got["out"]), ref["out"]) <= TOL_BF16
    P = f32_host(got["P"])
    refP = oracle.partial_sumsq(ref["h"], ops.rms_tile_width())
    assert norm_err(P, refP) <= 1e-5 * 10  # fp32 sums over 128 features vs exact


def test_mlp_tiny_config():
    w = inputs.make_workload("mlp_tiny")
    say("mlp_tiny (M=64 d=256 ffn=512)")
    got = run_fused(w)
    ref = oracle_rows(w)
    assert norm_err(bf16_host(got["h"]), ref["h"]) <= TOL_BF16
    assert row_rel_err(f32_host(got["r"]), ref["r"]) <= TOL_ROW
    assert norm_err(bf16_host(got["out"]), ref["out"]) <= TOL_BF16


@pytest.mark.parametrize("name", ["mlp_1b", "mlp_7b", "mlp_70b"])
def test_mlp_full_size_every_row(name):
    """Full MLP shapes at the 1B, 7B and 70B hidden sizes in the launch
    configuration the benchmark times; h, r and out of every row against the
    oracle (run over row chunks: every block is row-independent)."""
    w = inputs.make_workload(name)
    say(f"{name} full size {w.sizes}, every row")
    got = run_fused(w)
    h_all, out_all = bf16_host(got["h"]), bf16_host(got["out"])
    r_all = f32_host(got["r"])
    eh, eo, er = MaxErr(), MaxErr(), 0.0
    for rows in row_chunks(w.sizes["M"]):
        ref = oracle_rows(w, rows)
        eh.add(h_all[rows], ref["h"])
        eo.add(out_all[rows], ref["out"])
        er = max(er, row_rel_err(r_all[rows], ref["r"]))
    say(f"{name}: h {eh.value():.2e}, out {eo.value():.2e}, r {er:.2e}")
    assert eh.value() <= TOL_BF16
    assert eo.value() <= TOL_BF16
    assert er <= TOL_ROW


def test_fused_not_less_accurate_than_unfused():
    """The fused error against the oracle is no larger than the unfused
    sequence's (both on the GPU, same inputs)."""
    w = inputs.make_mlp(seed=5, M=512, d=1024, K1=1024, ffn=2048)
    say("fused vs unfused accuracy M=512 d=1024 ffn=2048")
    fz, uf = run_fused(w), run_unfused(w)
    ref = oracle_rows(w)
    e_f = norm_err(bf16_host(fz["out"]), ref["out"])
    e_u = norm_err(bf16_host(uf["out"]), ref["out"])
    say(f"fused {e_f:.3e} vs unfused {e_u:.3e}")
    assert e_u <= TOL_BF16 * 2
    assert e_f <= TOL_BF16
    assert e_f <= e_u, (e_f, e_u)

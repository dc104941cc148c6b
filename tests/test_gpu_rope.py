"""GPU parity of the attention-input block (GEMM1 residual/partial-RMS ->
reduce -> QKV GEMM with row-scale + RoPE epilogue) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, TOL_ROW, MaxErr, bf16_dev, bf16_host, dec_bf16, f32_dev, row_chunks,
                            f32_host, i32_dev, norm_err, row_rel_err, sample_rows, say)

pytestmark = pytest.mark.gpu
EPS = 1e-5


def run_fused(w, eps=EPS, max_pos=None):
    sz = w.sizes
    M, d, K1 = sz["M"], sz["d"], sz["K1"]
    nq, nkv, hd = sz["n_q"], sz["n_kv"], sz["head_dim"]
    max_pos = max_pos or sz["seq_len"]
    x, res, w1 = bf16_dev(w.arrays["x"]), bf16_dev(w.arrays["res"]), bf16_dev(w.arrays["w1"])
    wqkv = bf16_dev(w.arrays["wqkv"])
    gamma = f32_dev(w.arrays["gamma"])
    wqkv_f = torch.empty_like(wqkv)
    ops.fold_gamma(wqkv, gamma, wqkv_f)
    cos = torch.empty(max_pos, hd // 2, dtype=torch.float32, device=DEV)
    sin = torch.empty_like(cos)
    ops.rope_tables(sz["theta"], max_pos, hd, cos, sin)
    pos = i32_dev(w.arrays["pos"])
    h = torch.empty(M, d, dtype=torch.bfloat16, device=DEV)
    P = torch.empty(ops.rms_tiles(d), M, dtype=torch.float32, device=DEV)
    r = torch.empty(M, dtype=torch.float32, device=DEV)
    qkv = torch.empty(M, (nq + 2 * nkv) * hd, dtype=torch.bfloat16, device=DEV)
    ops.gemm_residual_partialrms(x, w1, res, h, P)
    ops.rms_reduce(P, d, eps, r)
    ops.gemm_rope(h, wqkv_f, r, cos, sin, pos, qkv, nq, nkv, hd)
    torch.cuda.synchronize()
    return {"h": h, "r": r, "qkv": qkv, "cos": cos, "sin": sin}


def oracle_rows(w, rows=None, eps=EPS, max_pos=None):
    sz = w.sizes
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    return oracle.attn_in_block(dec_bf16(sel(w.arrays["x"])), dec_bf16(sel(w.arrays["res"])),
                                dec_bf16(w.arrays["w1"]), dec_bf16(w.arrays["wqkv"]),
                                w.arrays["gamma"].astype(np.float64), eps, sel(w.arrays["pos"]),
                                sz["n_q"], sz["n_kv"], sz["head_dim"], sz["theta"],
                                max_pos or sz["seq_len"])


def test_rope_tables_match_oracle():
    say("rope tables theta=5e5 max_pos=2048 hd=64")
    cos = torch.empty(2048, 32, dtype=torch.float32, device=DEV)
    sin = torch.empty_like(cos)
    ops.rope_tables(500000.0, 2048, 64, cos, sin)
    torch.cuda.synchronize()
    rc, rs = oracle.rope_tables(2048, 64, 500000.0)
    # fp64 angles rounded once to fp32
    assert float(np.max(np.abs(f32_host(cos) - rc))) <= 6e-8
    assert float(np.max(np.abs(f32_host(sin) - rs))) <= 6e-8


@pytest.mark.parametrize("M,d,K1,nq,nkv,seq", [
    (300, 256, 192, 4, 2, 100),    # ragged M, many positions
    (200, 384, 128, 3, 1, 64),     # 5 heads: the last wave tile holds one head
    # head counts that are a multiple of 6 run on the 128 x 384 block tile
    (200, 256, 128, 4, 1, 64),     # 6 heads: one tile column, ragged M, four stages
    (300, 128, 128, 8, 2, 100),    # 12 heads: two tile columns, three row tiles, two stages
    (130, 64, 64, 2, 2, 50),       # 6 heads, one stage per tile
])
def test_rope_block_ragged(M, d, K1, nq, nkv, seq):
    w = inputs.make_attn(seed=7, M=M, d=d, K1=K1, n_q=nq, n_kv=nkv, head_dim=64, seq_len=seq)
    say(f"rope block M={M} d={d} K1={K1} nq={nq} nkv={nkv} seq={seq}")
    got = run_fused(w)
    ref = oracle_rows(w)
    assert norm_err(bf16_host(got["h"]), ref["h"]) <= TOL_BF16
    assert row_rel_err(f32_host(got["r"]), ref["r"]) <= TOL_ROW
    q = bf16_host(got["qkv"])
    assert norm_err(q, ref["qkv"]) <= TOL_BF16
    # the v heads are the plain row-scaled projection: check them separately
    vlo = (nq + nkv) * 64
    assert norm_err(q[:, vlo:], ref["qkv"][:, vlo:]) <= TOL_BF16


@pytest.mark.parametrize("M,d,K1,nq,nkv,seq", [
    (300, 256, 192, 4, 2, 100),    # 8 heads of 128: four tile columns, ragged M
    (200, 256, 128, 3, 1, 64),     # 5 heads: the last tile column holds one head
    (130, 128, 64, 8, 8, 50),      # 24 heads (no grouping), one stage per tile
])
def test_rope_block_head128(M, d, K1, nq, nkv, seq):
    """Heads of 128 (the 7B / 70B shapes): a wave's 128 features are one head
    and the rotate-half partner of feature c is c + 64."""
    w = inputs.make_attn(seed=11, M=M, d=d, K1=K1, n_q=nq, n_kv=nkv, head_dim=128, seq_len=seq)
    say(f"rope block hd=128 M={M} d={d} K1={K1} nq={nq} nkv={nkv} seq={seq}")
    got = run_fused(w)
    ref = oracle_rows(w)
    assert row_rel_err(f32_host(got["r"]), ref["r"]) <= TOL_ROW
    q = bf16_host(got["qkv"])
    assert norm_err(q, ref["qkv"]) <= TOL_BF16
    vlo = (nq + nkv) * 128
    assert norm_err(q[:, vlo:], ref["qkv"][:, vlo:]) <= TOL_BF16
    # rotated half of every q and k head on its own (a swapped pair would
    # still leave the unrotated half right)
    for hh in range(nq + nkv):
        c0 = hh * 128
        assert norm_err(q[:, c0 + 64:c0 + 128], ref["qkv"][:, c0 + 64:c0 + 128]) <= TOL_BF16


def test_rope_head128_chained_sampled_rows():
    """Heads of 128 at M = 16384 with 10 heads (5 tile columns): 320 tiles, so
    workgroups chain into a second tile; sampled rows vs the oracle."""
    w = inputs.make_attn(seed=12, M=16384, d=128, K1=64, n_q=8, n_kv=1, head_dim=128,
                         seq_len=2048)
    say("rope block hd=128, chained tiles (M=16384, 10 heads)")
    got = run_fused(w)
    rows = sample_rows(w.sizes["M"], n=48)
    ref = oracle_rows(w, rows)
    assert norm_err(bf16_host(got["qkv"][rows.tolist()]), ref["qkv"]) <= TOL_BF16


@pytest.mark.parametrize("hd", [64, 128])
def test_rope_position_zero_identity_any_head(hd):
    """Positions all 0 with heads of 64 and 128 on the 256 x 256 tile."""
    w = inputs.make_attn(seed=13, M=96, d=128, K1=64, n_q=2, n_kv=1, head_dim=hd, seq_len=1)
    say(f"rope block, all positions 0, hd={hd}")
    got = run_fused(w)
    ref = oracle_rows(w)
    n = oracle.rmsnorm(ref["h"], w.arrays["gamma"].astype(np.float64), EPS)
    plain = oracle.gemm_nt(n, dec_bf16(w.arrays["wqkv"]))
    assert norm_err(bf16_host(got["qkv"]), plain) <= TOL_BF16


@pytest.mark.parametrize("nq,nkv", [(2, 1), (4, 1)])  # 4 heads; 6 heads (128 x 384 tile)
def test_rope_position_zero_is_identity_on_gpu(nq, nkv):
    """With every position 0 the rotation is the identity, so q|k|v equal the
    plain row-scaled projection (checked against the oracle with RoPE off)."""
    w = inputs.make_attn(seed=8, M=128, d=256, K1=128, n_q=nq, n_kv=nkv, head_dim=64, seq_len=1)
    say(f"rope block, all positions 0, nq={nq} nkv={nkv}")
    got = run_fused(w)
    ref = oracle_rows(w)
    n = oracle.rmsnorm(ref["h"], w.arrays["gamma"].astype(np.float64), EPS)
    plain = oracle.gemm_nt(n, dec_bf16(w.arrays["wqkv"]))
    assert norm_err(bf16_host(got["qkv"]), plain) <= TOL_BF16


def test_attn_rope_full_every_row():
    """Full attention-input shape (M=8192, d=2048, GEMM1 K=8192, 32 q / 8 kv
    heads of 64, theta=5e5, positions m mod 2048); h, r and qkv of every row
    against the oracle (over row chunks)."""
    w = inputs.make_workload("attn_rope")
    say("attn_rope full size, every row")
    got = run_fused(w)
    h_all, q_all = bf16_host(got["h"]), bf16_host(got["qkv"])
    r_all = f32_host(got["r"])
    eh, eq, er = MaxErr(), MaxErr(), 0.0
    for rows in row_chunks(w.sizes["M"]):
        ref = oracle_rows(w, rows)
        eh.add(h_all[rows], ref["h"])
        eq.add(q_all[rows], ref["qkv"])
        er = max(er, row_rel_err(r_all[rows], ref["r"]))
    say(f"attn_rope: h {eh.value():.2e}, qkv {eq.value():.2e}, r {er:.2e}")
    assert eh.value() <= TOL_BF16
    assert er <= TOL_ROW
    assert eq.value() <= TOL_BF16


def test_rope_wide_tile_chained_sampled_rows():
    """18 heads (QKV width 1152, three 128 x 384 tile columns) at M = 16384:
    384 tiles for the compute units, so workgroups chain into a second tile;
    sampled rows vs the oracle."""
    w = inputs.make_attn(seed=9, M=16384, d=128, K1=64, n_q=12, n_kv=3, head_dim=64,
                         seq_len=2048)
    say("rope block, 128 x 384 tiles chained (M=16384, 18 heads)")
    got = run_fused(w)
    rows = sample_rows(w.sizes["M"], n=48)
    ref = oracle_rows(w, rows)
    assert norm_err(bf16_host(got["h"][rows.tolist()]), ref["h"]) <= TOL_BF16
    assert norm_err(bf16_host(got["qkv"][rows.tolist()]), ref["qkv"]) <= TOL_BF16

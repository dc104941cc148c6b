"""Degenerate numeric cases of the epilogues on the GPU, against the oracle:
SwiGLU (forward and backward) far into the saturated ranges of the sigmoid
(exp overflows to inf / underflows to 0), all-zero token rows (h = 0, so
r = eps^-1/2 and out = 0), and LM-head logits of large magnitude (the block
log-sum-exp must stay finite)."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, TOL_ROW, bf16_dev, bf16_host, dec_bf16, f32_dev,
                            f32_host, norm_err, row_rel_err, say)

pytestmark = pytest.mark.gpu


def _bf(rng, shape, std):
    return inputs.to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def test_swiglu_saturated_sigmoid():
    """Pre-activations with standard deviation ~100: about half of the gate
    values lie beyond +-88 where exp overflows or underflows in fp32."""
    rng = np.random.default_rng(11)
    M, K, N = 512, 256, 512
    x, wg, wu = _bf(rng, (M, K), 1.0), _bf(rng, (N, K), 100.0 / 16), _bf(rng, (N, K), 1.0 / 16)
    r = np.ones(M, dtype=np.float32)
    say("swiglu with saturated sigmoid M=512 K=256 N=512")
    out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    ops.gemm_rowscale_swiglu(bf16_dev(x), bf16_dev(wg), bf16_dev(wu), f32_dev(r), out)
    torch.cuda.synchronize()
    g = oracle.gemm_nt(dec_bf16(x), dec_bf16(wg))
    u = oracle.gemm_nt(dec_bf16(x), dec_bf16(wu))
    assert float(np.mean(np.abs(g) > 88.0)) > 0.3  # the case really saturates
    got = bf16_host(out)
    assert np.all(np.isfinite(got))
    assert norm_err(got, oracle.swiglu(g, u)) <= TOL_BF16


def test_swiglu_bwd_saturated_sigmoid():
    """The SwiGLU-backward epilogue with saved pre-activations g of magnitude
    up to several hundred (sigmoid exactly 0 or 1 in fp32)."""
    rng = np.random.default_rng(12)
    M, d, ffn = 512, 256, 512
    dy, wdT = _bf(rng, (M, d), 1.0), _bf(rng, (ffn, d), 1.0 / 16)
    g = (rng.standard_normal((M, ffn)) * 150).astype(np.float32)
    u = rng.standard_normal((M, ffn)).astype(np.float32)
    gu = inputs.to_bf16_bits(np.concatenate([g, u], axis=1))
    say("swiglu backward with saturated sigmoid M=512 d=256 ffn=512")
    dz = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=DEV)
    pdot = torch.empty(ops.rms_tiles(ffn), M, dtype=torch.float32, device=DEV)
    ops.gemm_swiglu_bwd(bf16_dev(dy), bf16_dev(wdT), bf16_dev(gu), dz, pdot)
    torch.cuda.synchronize()
    gq = dec_bf16(gu)
    dout = oracle.gemm_nt(dec_bf16(dy), dec_bf16(wdT))
    dg, du = oracle.swiglu_grad(dout, gq[:, :ffn], gq[:, ffn:])
    got = bf16_host(dz)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(f32_host(pdot)))
    assert norm_err(got[:, :ffn], dg) <= TOL_BF16
    assert norm_err(got[:, ffn:], du) <= TOL_BF16


def test_zero_rows():
    """Token rows whose input and residual are zero: h = 0, the partial sums
    are 0, r = eps^-1/2 and the block output is exactly 0 on those rows."""
    w = inputs.make_mlp(seed=13, M=300, d=256, K1=256, ffn=512)
    zero = np.arange(0, 300, 7)
    for k in ("x", "res"):
        w.arrays[k] = w.arrays[k].copy()
        w.arrays[k][zero] = 0
    say("mlp block with all-zero rows M=300 d=256 ffn=512")
    from tests.test_gpu_mlp import oracle_rows, run_fused
    got = run_fused(w)
    ref = oracle_rows(w)
    r = f32_host(got["r"])
    assert row_rel_err(r, ref["r"]) <= TOL_ROW
    assert np.allclose(r[zero], 1.0 / np.sqrt(1e-5), rtol=1e-6)
    out = bf16_host(got["out"])
    assert np.all(out[zero] == 0.0)
    assert norm_err(out, ref["out"]) <= TOL_BF16


def test_lse_large_logits():
    """Logits of magnitude ~100: every tile's max dominates its sum of
    exponentials; the merged loss stays finite and matches the oracle."""
    rng = np.random.default_rng(14)
    M, K, V = 512, 128, 4096
    x, wl = _bf(rng, (M, K), 1.0), _bf(rng, (V, K), 100.0 / np.sqrt(K))
    labels = rng.integers(0, V, size=M).astype(np.int32)
    say("block lse with logits of magnitude ~100 M=512 K=128 V=4096")
    T = ops.lse_tiles(V)
    tmax = torch.empty(T, M, dtype=torch.float32, device=DEV)
    tsum = torch.empty_like(tmax)
    zl, loss = (torch.empty(M, dtype=torch.float32, device=DEV) for _ in range(2))
    ops.gemm_block_lse(bf16_dev(x), bf16_dev(wl), torch.from_numpy(labels).to(DEV), tmax, tsum,
                       zl, loss)
    torch.cuda.synchronize()
    ref = oracle.lm_head_ce(dec_bf16(x), dec_bf16(wl), labels)
    got = f32_host(loss)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(ref["loss"]))) > 100.0
    err = np.abs(got - ref["loss"])
    worst = int(np.argmax(err / np.abs(ref["loss"])))
    say(f"worst relative row {worst}: loss {ref['loss'][worst]:.3e} got {got[worst]:.3e} "
        f"lse {ref['lse'][worst]:.3f}; max err / |lse| {float(np.max(err / np.abs(ref['lse']))):.2e}")
    # loss = lse - z_label cancels when the label is (near) the arg max, so its
    # error is bounded relative to |lse| (the fp32 values being subtracted),
    # and relative to the loss itself where the loss is not small
    assert float(np.max(err / np.abs(ref["lse"]))) <= TOL_ROW
    big = np.abs(ref["loss"]) >= 1.0
    assert row_rel_err(got[big], ref["loss"][big]) <= TOL_ROW

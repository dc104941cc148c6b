"""The plain GEMM with a split reduction (coda_gemm_bf16_splitk), used for the
weight gradients whose d x d outputs have too few tiles to occupy the GPU.

Integer-valued inputs keep every partial and final sum exact in fp32, so the
bf16 result is compared bit for bit with the oracle's product rounded by the
oracle's bf16 encoder; random inputs are compared at the bf16 tolerance,
including the weight-gradient shape dWo = dh^T x (2048 x 2048, 8192 tokens)."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, bf16_dev, bf16_encode_few, bf16_host, dec_bf16,
                            norm_err, say)

pytestmark = pytest.mark.gpu


def _ints(rng, shape):
    return rng.integers(-1, 2, size=shape).astype(np.float32)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run(A, W, parts, ws=None):
    M, N = A.shape[0], W.shape[0]
    C = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    if ws is None:
        ws = torch.empty(parts, M, N, dtype=torch.float32, device=DEV)
    ops.gemm_bf16_splitk(A, W, C, ws)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("M,N,K,parts", [
    (2048, 2048, 8192, 4),   # the dWo launch of the 1B backward, bit for bit
    (2048, 2048, 1024, 4),   # 64 tiles x 4 parts: one work unit per compute unit
    (4096, 4096, 512, 2),    # 512 units: workgroups chain units of different parts
    (520, 2048, 8192, 16),   # 384 units of 512 columns, ragged last tile row
    (300, 272, 256, 4),      # ragged rows and columns, one stage per part
    (1, 16, 128, 2),         # a single row and a single 16-wide feature group
    (257, 272, 192, 1),      # one part: the plain GEMM through the workspace
])
def test_splitk_exact(M, N, K, parts):
    rng = np.random.default_rng(M * 7 + N + K + parts)
    a, w = _ints(rng, (M, K)), _ints(rng, (N, K))
    say(f"split-K exact M={M} N={N} K={K} parts={parts}")
    C = _run(bf16_dev(inputs.to_bf16_bits(a)), bf16_dev(inputs.to_bf16_bits(w)), parts)
    y = oracle.gemm_nt(a, w)
    assert np.array_equal(_bits(C), bf16_encode_few(y))


def test_splitk_workspace_reuse_and_determinism():
    """A second call on a smaller shape overwrites the parts it reads (no
    clearing), and repeated calls give the same bits."""
    rng = np.random.default_rng(11)
    ws = torch.empty(4, 1024, 1024, dtype=torch.float32, device=DEV)
    ws.fill_(float("nan"))
    big = [bf16_dev(inputs.to_bf16_bits(rng.standard_normal((1024, 2048)).astype(np.float32)))
           for _ in range(2)]
    say("split-K workspace reuse 1024x1024x2048 then 300x528x1024")
    C1 = _run(big[0], big[1], 4, ws)
    C1b = _run(big[0], big[1], 4, ws)
    assert torch.equal(_bits_t(C1), _bits_t(C1b))
    a, w = _ints(rng, (300, 1024)), _ints(rng, (528, 1024))
    small_ws = ws.view(-1)[:4 * 300 * 528].view(4, 300, 528)
    C2 = _run(bf16_dev(inputs.to_bf16_bits(a)), bf16_dev(inputs.to_bf16_bits(w)), 4, small_ws)
    assert np.array_equal(_bits(C2), bf16_encode_few(oracle.gemm_nt(a, w)))


def _bits_t(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("parts", [4, 8])
def test_splitk_weight_gradient_shape_sampled(parts):
    """dWo = dh^T x at the 1B MLP shape: A = dh^T [2048, 8192 tokens],
    W = x^T [2048, 8192]; sampled output rows against the fp64 oracle, and the
    whole output against the unsplit GEMM (both within the bf16 tolerance)."""
    rng = np.random.default_rng(100 + parts)
    d, T = 2048, 8192
    a_bits = inputs.to_bf16_bits(rng.standard_normal((d, T)).astype(np.float32))
    w_bits = inputs.to_bf16_bits(rng.standard_normal((d, T)).astype(np.float32))
    A, W = bf16_dev(a_bits), bf16_dev(w_bits)
    say(f"split-K dWo shape 2048x2048x8192 parts={parts}")
    C = _run(A, W, parts)
    rows = np.arange(3, d, 61)
    ref = oracle.gemm_nt(dec_bf16(a_bits[rows]), dec_bf16(w_bits))
    assert norm_err(bf16_host(C)[rows], ref) <= TOL_BF16
    C0 = torch.empty_like(C)
    ops.gemm_bf16(A, W, C0)
    torch.cuda.synchronize()
    assert norm_err(bf16_host(C), bf16_host(C0)) <= TOL_BF16

"""GPU parity of the unfused baseline pieces that only the speed comparison
uses (in-place RoPE on a stored qkv, cross entropy of stored logits) against
the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, TOL_ROW, bf16_dev, bf16_host, dec_bf16, f32_dev,
                            f32_host, i32_dev, norm_err, row_rel_err, say)

pytestmark = pytest.mark.gpu


def test_rope_apply_vs_oracle():
    M, nq, nkv, hd, max_pos = 300, 4, 2, 64, 64
    N = (nq + 2 * nkv) * hd
    rng = np.random.default_rng(5)
    y = rng.standard_normal((M, N)).astype(np.float32)
    bits = inputs.to_bf16_bits(y)
    pos = (np.arange(M) * 7 % max_pos).astype(np.int32)
    cos, sin = oracle.rope_tables(max_pos, hd, 10000.0)
    say(f"rope_apply M={M} heads {nq}+{nkv}+{nkv}")
    qkv = bf16_dev(bits)
    ops.rope_apply(qkv, f32_dev(cos), f32_dev(sin), i32_dev(pos), nq, nkv, hd)
    torch.cuda.synchronize()
    ref = oracle.apply_rope(dec_bf16(bits), pos, nq + nkv, hd, cos.astype(np.float32).astype(np.float64),
                            sin.astype(np.float32).astype(np.float64))
    got = bf16_host(qkv)
    assert norm_err(got, ref) <= TOL_BF16
    # v heads untouched, bit for bit
    v0 = (nq + nkv) * hd
    assert np.array_equal(got[:, v0:], dec_bf16(bits)[:, v0:])


@pytest.mark.parametrize("M,V", [(64, 1008), (5, 128256)])
def test_cross_entropy_rows_vs_oracle(M, V):
    rng = np.random.default_rng(M + V)
    z = (rng.standard_normal((M, V)) * 3).astype(np.float32)
    bits = inputs.to_bf16_bits(z)
    labels = rng.integers(0, V, size=M).astype(np.int32)
    say(f"cross_entropy_rows M={M} V={V}")
    lse = torch.empty(M, dtype=torch.float32, device=DEV)
    loss = torch.empty_like(lse)
    ops.cross_entropy_rows(bf16_dev(bits), i32_dev(labels), lse, loss)
    torch.cuda.synchronize()
    zd = dec_bf16(bits)
    ref_lse = oracle.logsumexp_rows(zd)
    ref_loss = ref_lse - zd[np.arange(M), labels]
    assert row_rel_err(f32_host(lse), ref_lse) <= TOL_ROW
    assert np.max(np.abs(f32_host(loss) - ref_loss)) <= TOL_ROW * np.max(np.abs(ref_lse))

"""The LM-head entry point that allocates nothing (its partials in the
library's static scratch) against coda_gemm_block_lse with caller workspace,
through the C ABI: two calls in a row on one GPU, the second with a smaller
input, each giving the same lse and loss bit for bit (the same kernels and
launches), and the smaller one against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_ROW, bf16_dev, dec_bf16, f32_host, i32_dev, row_rel_err,
                            say)

pytestmark = pytest.mark.gpu


def _both(w, labels):
    M, V = w.sizes["M"], w.sizes["V"]
    x, wl, lab = bf16_dev(w.arrays["x"]), bf16_dev(w.arrays["wlm"]), i32_dev(labels)
    T = ops.lse_tiles(V)
    tmax = torch.empty(T, M, dtype=torch.float32, device=DEV)
    tsum = torch.empty_like(tmax)
    zl = torch.empty(M, dtype=torch.float32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    loss_w, lse_w = torch.empty(M, **f32), torch.empty(M, **f32)
    loss_n, lse_n = torch.full((M,), float("nan"), **f32), torch.full((M,), float("nan"), **f32)
    ops.gemm_block_lse(x, wl, lab, tmax, tsum, zl, loss_w, lse=lse_w)
    ops.gemm_block_lse_noalloc(x, wl, lab, loss_n, lse=lse_n)
    torch.cuda.synchronize()
    return (f32_host(loss_w), f32_host(lse_w)), (f32_host(loss_n), f32_host(lse_n))


def test_noalloc_lse_two_calls_second_smaller():
    # first call: the full LM-head shape (the largest input the scratch holds)
    w1 = inputs.make_workload("lm_head")
    say("no-alloc block lse, call 1: M=8192 d=2048 V=128256")
    (lw, sw), (ln, sn) = _both(w1, w1.arrays["labels"])
    assert np.array_equal(ln, lw) and np.array_equal(sn, sw)
    # second call, smaller and ragged, with ignored labels: the scratch still
    # holds the first call's partials, which must not leak into this result
    w2 = inputs.make_lm(seed=33, M=300, d=192, V=1008)
    lab = w2.arrays["labels"].copy()
    lab[[3, 77]] = [-100, 1008]
    say("no-alloc block lse, call 2: M=300 d=192 V=1008")
    (lw, sw), (ln, sn) = _both(w2, lab)
    assert np.array_equal(ln, lw) and np.array_equal(sn, sw)
    ref = oracle.lm_head_ce(dec_bf16(w2.arrays["x"]), dec_bf16(w2.arrays["wlm"]), lab)
    assert row_rel_err(sn, ref["lse"]) <= TOL_ROW
    keep = np.setdiff1d(np.arange(300), [3, 77])
    assert row_rel_err(ln[keep], ref["loss"][keep]) <= TOL_ROW
    assert ln[3] == 0.0 and ln[77] == 0.0


def test_noalloc_lse_rejects_sizes_past_the_scratch():
    """Sizes whose partials exceed the scratch are rejected before any launch."""
    M, V, K = 16384, 128256, 64
    x = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    wl = torch.empty(V, K, dtype=torch.bfloat16, device=DEV)
    lab = torch.zeros(M, dtype=torch.int32, device=DEV)
    loss = torch.empty(M, dtype=torch.float32, device=DEV)
    with pytest.raises(ops.CodaError) as e:
        ops.gemm_block_lse_noalloc(x, wl, lab, loss)
    assert e.value.status == -2

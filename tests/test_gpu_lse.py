"""GPU parity of the LM-head cross entropy (GEMM with block log-sum-exp
epilogue + merge) against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_ROW, bf16_dev, dec_bf16, f32_dev, f32_host, i32_dev,
                            row_rel_err, sample_rows, say)

pytestmark = pytest.mark.gpu


def run_lse(w, r=None, W=None, labels=None):
    M, d, V = w.sizes["M"], w.sizes["d"], w.sizes["V"]
    x = bf16_dev(w.arrays["x"])
    wl = W if W is not None else bf16_dev(w.arrays["wlm"])
    lab = i32_dev(w.arrays["labels"] if labels is None else labels)
    T = ops.lse_tiles(V)
    tmax = torch.empty(T, M, dtype=torch.float32, device=DEV)
    tsum = torch.empty_like(tmax)
    zl = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.empty(M, dtype=torch.float32, device=DEV)
    loss = torch.empty(M, dtype=torch.float32, device=DEV)
    ops.gemm_block_lse(x, wl, lab, tmax, tsum, zl, loss, lse=lse,
                       r=None if r is None else f32_dev(r))
    torch.cuda.synchronize()
    return {"tmax": f32_host(tmax), "tsum": f32_host(tsum), "zl": f32_host(zl),
            "lse": f32_host(lse), "loss": f32_host(loss)}


def oracle_rows(w, rows=None, r=None, labels=None, chunk=256):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    rr = None if r is None else sel(r).astype(np.float64)
    lab = w.arrays["labels"] if labels is None else labels
    return oracle.lm_head_ce(dec_bf16(sel(w.arrays["x"])), dec_bf16(w.arrays["wlm"]),
                             sel(lab), r=rr, chunk=chunk)


def check_partials(w, got, rows):
    """(max, sum-exp) pairs are not unique, so check what is: each tile's
    mx + ln(se) is that tile's own log-sum-exp, and re-merging the GPU's
    pairs on the host in several orders gives the row's lse."""
    wt = ops.lse_tile_width()
    x = dec_bf16(w.arrays["x"][rows])
    z = oracle.gemm_nt(x, dec_bf16(w.arrays["wlm"]))
    T = got["tmax"].shape[0]
    tl = got["tmax"][:, rows] + np.log(got["tsum"][:, rows])
    for t in range(T):
        ref = oracle.logsumexp_rows(z[:, t * wt:(t + 1) * wt])
        assert float(np.max(np.abs(tl[t] - ref))) <= 2e-5, t
    full = oracle.logsumexp_rows(z)
    mx, se = got["tmax"][:, rows], got["tsum"][:, rows]
    rng = np.random.default_rng(0)
    for order in (None, list(range(T))[::-1], list(rng.permutation(T))):
        assert float(np.max(np.abs(oracle.lse_merge(mx, se, order) - full))) <= 2e-5


def test_lse_ragged_small():
    w = inputs.make_lm(seed=11, M=300, d=192, V=1008)
    say("block lse M=300 d=192 V=1008 (last tile 112 wide)")
    got = run_lse(w)
    ref = oracle_rows(w)
    assert row_rel_err(got["loss"], ref["loss"]) <= TOL_ROW
    assert row_rel_err(got["lse"], ref["lse"]) <= TOL_ROW
    assert float(np.max(np.abs(got["zl"] - ref["label_logit"]))) <= 1e-4
    check_partials(w, got, np.arange(300))


def test_lse_with_row_scale():
    w = inputs.make_lm(seed=12, M=257, d=128, V=512)
    r = np.random.default_rng(3).uniform(0.5, 2.0, size=257).astype(np.float32)
    say("block lse with row scale M=257 d=128 V=512")
    got = run_lse(w, r=r)
    ref = oracle_rows(w, r=r)
    assert row_rel_err(got["loss"], ref["loss"]) <= TOL_ROW


def test_lse_zero_weights_gives_ln_v():
    """W = 0: all logits are 0, so every row's loss is ln V exactly."""
    w = inputs.make_lm(seed=13, M=130, d=64, V=1008)
    say("block lse with zero weights")
    W0 = torch.zeros(1008, 64, dtype=torch.bfloat16, device=DEV)
    got = run_lse(w, W=W0)
    assert float(np.max(np.abs(got["loss"] - math.log(1008)))) <= 1e-5
    assert float(np.max(np.abs(got["zl"]))) == 0.0


def test_lse_ignored_labels():
    """Labels outside [0, V) (an ignore index of -100, and V or more) mark rows
    that carry no loss: loss 0 on those rows in the fused path and in the
    unfused row cross entropy, lse still the row's log-sum-exp, every other
    row unchanged (the label-logit buffer starts as NaN, so a read of an
    unwritten entry would show)."""
    w = inputs.make_lm(seed=14, M=300, d=192, V=1008)
    lab = w.arrays["labels"].copy()
    ign = np.array([0, 5, 17, 128, 255, 299])
    lab[ign] = [-100, -1, 1008, 5000, -100, 2 ** 31 - 1]
    say("block lse with ignored labels M=300 d=192 V=1008")
    got = run_lse(w, labels=lab)
    ref = oracle_rows(w, labels=lab)
    keep = np.setdiff1d(np.arange(300), ign)
    assert np.all(got["loss"][ign] == 0.0)
    assert row_rel_err(got["loss"][keep], ref["loss"][keep]) <= TOL_ROW
    assert row_rel_err(got["lse"], ref["lse"]) <= TOL_ROW
    assert np.all(np.isnan(got["zl"][ign]))
    # the unfused baseline: stored bf16 logits, then the row cross entropy
    M, V = 300, 1008
    x, wl = bf16_dev(w.arrays["x"]), bf16_dev(w.arrays["wlm"])
    z = torch.empty(M, V, dtype=torch.bfloat16, device=DEV)
    lse_u = torch.empty(M, dtype=torch.float32, device=DEV)
    loss_u = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    ops.gemm_bf16(x, wl, z)
    ops.cross_entropy_rows(z, i32_dev(lab), lse_u, loss_u)
    torch.cuda.synchronize()
    lu = f32_host(loss_u)
    assert np.all(lu[ign] == 0.0)
    assert float(np.max(np.abs(lu[keep] - ref["loss"][keep]))) <= 0.05  # bf16 logits
    assert float(np.max(np.abs(f32_host(lse_u) - ref["lse"]))) <= 0.05


def test_lm_head_full_every_row():
    """Full LM-head shape (M=8192, d=2048, V=128256) in the launch the
    benchmark times: the loss and lse of every row against the oracle, and the
    partial invariants on 64 rows."""
    w = inputs.make_workload("lm_head")
    say("lm_head full size, every row")
    got = run_lse(w)
    ref = oracle_rows(w, chunk=512)
    assert row_rel_err(got["loss"], ref["loss"]) <= TOL_ROW
    assert row_rel_err(got["lse"], ref["lse"]) <= TOL_ROW
    assert float(np.max(np.abs(got["zl"] - ref["label_logit"]))) <= 1e-3
    rows = sample_rows(w.sizes["M"], n=64)
    check_partials(w, got, rows)

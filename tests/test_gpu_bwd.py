"""GPU parity of the MLP sub-layer backward (SwiGLU-backward GEMM ->
row-coefficient reduce -> RMSNorm-backward GEMM -> dx GEMM) and of the
forward variant that saves the pre-activations, against the CPU oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, bf16_dev, bf16_encode_few, bf16_host, dec_bf16,
                            f32_dev, f32_host, norm_err, sample_rows, say)

pytestmark = pytest.mark.gpu
EPS = 1e-5


def _ints(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def prep_weights(w):
    """Device weights: gamma folded into gate/up, and the transposed copies
    the backward GEMMs read (WdT = Wd^T, W2T = [Wg'; Wu']^T, WoT = Wo^T)."""
    d, K1, ffn = (w.sizes[k] for k in ("d", "K1", "ffn"))
    wo, wg, wu, wd = (bf16_dev(w.arrays[k]) for k in ("w1", "wg", "wu", "wd"))
    gamma = f32_dev(w.arrays["gamma"])
    wg_f, wu_f = torch.empty_like(wg), torch.empty_like(wu)
    ops.fold_gamma(wg, gamma, wg_f)
    ops.fold_gamma(wu, gamma, wu_f)
    WdT = torch.empty(ffn, d, dtype=torch.bfloat16, device=DEV)
    ops.transpose(wd, WdT)
    W2T = torch.empty(d, 2 * ffn, dtype=torch.bfloat16, device=DEV)
    ops.transpose(wg_f, W2T[:, :ffn])
    ops.transpose(wu_f, W2T[:, ffn:])
    WoT = torch.empty(K1, d, dtype=torch.bfloat16, device=DEV)
    ops.transpose(wo, WoT)
    return dict(wo=wo, wg_f=wg_f, wu_f=wu_f, WdT=WdT, W2T=W2T, WoT=WoT)


def run_fused(w, eps=EPS):
    """Forward (saving z) and backward of the sub-layer on the GPU."""
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    p = prep_weights(w)
    x, res, dy = (bf16_dev(w.arrays[k]) for k in ("x", "res", "dy"))
    h = torch.empty(M, d, dtype=torch.bfloat16, device=DEV)
    P = torch.empty(ops.rms_tiles(d), M, dtype=torch.float32, device=DEV)
    r = torch.empty(M, dtype=torch.float32, device=DEV)
    out = torch.empty(M, ffn, dtype=torch.bfloat16, device=DEV)
    gu = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=DEV)
    ops.gemm_residual_partialrms(x, p["wo"], res, h, P)
    ops.rms_reduce(P, d, eps, r)
    ops.gemm_rowscale_swiglu_save(h, p["wg_f"], p["wu_f"], r, out, gu)
    dz = torch.full((M, 2 * ffn), float("nan"), dtype=torch.bfloat16, device=DEV)
    pdot = torch.full((ops.rms_tiles(ffn), M), float("nan"), dtype=torch.float32, device=DEV)
    c = torch.empty(M, dtype=torch.float32, device=DEV)
    dh = torch.full((M, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(M, K1, dtype=torch.bfloat16, device=DEV)
    ops.gemm_swiglu_bwd(dy, p["WdT"], gu, dz, pdot)
    ops.rms_bwd_reduce(pdot, d, r, c)
    ops.gemm_rmsnorm_bwd(dz, p["W2T"], h, dy, r, c, dh)
    ops.gemm_bf16(dh, p["WoT"], dx)
    torch.cuda.synchronize()
    return dict(h=h, r=r, out=out, gu=gu, dz=dz, pdot=pdot, c=c, dh=dh, dx=dx, **p)


def run_unfused(w, fz, eps=EPS):
    """The unfused backward on the GPU from the fused forward's h, r and gu:
    plain GEMM -> SwiGLU backward pass -> plain GEMM -> RMSNorm backward pass
    -> plain GEMM, each result through HBM."""
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    dy = bf16_dev(w.arrays["dy"])
    dout = torch.empty(M, ffn, dtype=torch.bfloat16, device=DEV)
    dz = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=DEV)
    G = torch.empty(M, d, dtype=torch.bfloat16, device=DEV)
    dh = torch.empty(M, d, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(M, K1, dtype=torch.bfloat16, device=DEV)
    ops.gemm_bf16(dy, fz["WdT"], dout)
    ops.swiglu_bwd(dout, fz["gu"], dz)
    ops.gemm_bf16(dz, fz["W2T"], G)
    ops.rmsnorm_bwd(G, fz["h"], dy, eps, dh)
    ops.gemm_bf16(dh, fz["WoT"], dx)
    torch.cuda.synchronize()
    return dict(dz=dz, dh=dh, dx=dx)


def oracle_rows(w, rows=None, eps=EPS):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    return oracle.mlp_layer_bwd(dec_bf16(sel(w.arrays["x"])), dec_bf16(sel(w.arrays["res"])),
                                dec_bf16(w.arrays["w1"]), dec_bf16(w.arrays["wg"]),
                                dec_bf16(w.arrays["wu"]), w.arrays["gamma"].astype(np.float64),
                                eps, dec_bf16(w.arrays["wd"]), dec_bf16(sel(w.arrays["dy"])))


def check_against_oracle(got, ref, rows=None, w=None):
    sel = (lambda t: t) if rows is None else (lambda t: t[rows.tolist()])
    ffn = ref["dg"].shape[1]
    dz = bf16_host(sel(got["dz"]))
    errs = {"dg": norm_err(dz[:, :ffn], ref["dg"]), "du": norm_err(dz[:, ffn:], ref["du"]),
            "dh": norm_err(bf16_host(sel(got["dh"])), ref["dh"]),
            "dx": norm_err(bf16_host(sel(got["dx"])), ref["dx"])}
    if "c" in got:
        c = f32_host(got["c"])
        errs["c"] = norm_err(c if rows is None else c[rows], ref["coef"])
    say(f"errors {errs}")
    for k, e in errs.items():
        assert e <= TOL_BF16, (k, e)


def test_transpose_exact():
    rng = np.random.default_rng(0)
    for rows, cols in ((1, 1), (70, 130), (257, 64), (64, 1000), (136, 200), (8, 8), (264, 392),
                       (1032, 136)):
        say(f"transpose {rows}x{cols}")
        a = bf16_dev(inputs.to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32)))
        dst = torch.zeros(cols, rows + 24, dtype=torch.bfloat16, device=DEV)
        ops.transpose(a, dst[:, 8:8 + rows])
        torch.cuda.synchronize()
        assert torch.equal(dst[:, 8:8 + rows].cpu(), a.t().cpu())
        assert not dst[:, :8].any().item() and not dst[:, 8 + rows:].any().item()


def test_transpose_full_size_exact():
    """The token-major copies at the 1B backward sizes: dz [8192, 16384] and
    the row-scaled h [8192, 2048], bit for bit (the scaled copy against the
    fp32 product rounded to bf16 with round-to-nearest-even, as the kernel
    computes it; torch's float -> bfloat16 conversion rounds the same way)."""
    g = torch.Generator(device=DEV).manual_seed(5)
    say("transpose full size dz 8192x16384")
    dz = torch.randn(8192, 16384, device=DEV, generator=g).to(torch.bfloat16)
    dzT = torch.empty(16384, 8192, dtype=torch.bfloat16, device=DEV)
    ops.transpose(dz, dzT)
    torch.cuda.synchronize()
    assert torch.equal(dzT.view(torch.int16), dz.t().contiguous().view(torch.int16))
    del dz, dzT
    say("scaled transpose full size h 8192x2048")
    h = torch.randn(8192, 2048, device=DEV, generator=g).to(torch.bfloat16)
    r = torch.rand(8192, device=DEV, generator=g) + 0.5
    hT = torch.empty(2048, 8192, dtype=torch.bfloat16, device=DEV)
    ops.transpose(h, hT, row_scale=r)
    torch.cuda.synchronize()
    ref = (h.float() * r[:, None]).to(torch.bfloat16).t().contiguous()
    assert torch.equal(hT.view(torch.int16), ref.view(torch.int16))


def test_forward_save_matches_forward():
    """The saving variant stores the same out bits as the plain GEMM2 and
    g, u of the oracle."""
    w = inputs.make_mlp_bwd(seed=2, M=600, d=448, K1=320, ffn=1056)
    say("forward save M=600 d=448 ffn=1056")
    got = run_fused(w)
    out2 = torch.empty_like(got["out"])
    ops.gemm_rowscale_swiglu(got["h"], got["wg_f"], got["wu_f"], got["r"], out2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), got["out"].view(torch.int16))
    ref = oracle_rows(w)
    gu = bf16_host(got["gu"])
    assert norm_err(gu[:, :1056], ref["g"]) <= TOL_BF16
    assert norm_err(gu[:, 1056:], ref["u"]) <= TOL_BF16


@pytest.mark.parametrize("M,d,ffn", [
    (300, 320, 1056),    # ragged M and N, several tiles each way
    (8192, 2048, 4096),  # 512 SwiGLU-backward tiles: every workgroup chains
    (4096, 4096, 32),    # RMSNorm backward: one K stage per tile, 256 tiles
    (16384, 4096, 64),   # RMSNorm backward: two stages per tile, 1024 tiles
    (1, 64, 32),         # one token row, the smallest widths (one stage, one partial tile)
])
def test_bwd_epilogues_exact(M, d, ffn):
    """Values chosen so that every step is exact in fp32 (the bf16 stores
    then round the same exact values as the oracle's encoder): dY, Wd, W' in
    {-1,0,1}, g in {0, 64} (sigmoid exactly 1/2, and 1 in fp32 and fp64),
    u, h small integers, r = 1, c = 1/2.  dz, the partial sums and dh must
    equal the oracle's values bit for bit, which pins the epilogues' data
    layout."""
    rng = np.random.default_rng(M + d + ffn)
    dy, wdT = _ints(rng, (M, d), -1, 1), _ints(rng, (ffn, d), -1, 1)
    g = 64.0 * rng.integers(0, 2, size=(M, ffn)).astype(np.float32)
    u = _ints(rng, (M, ffn), -1, 2)
    say(f"exact backward epilogues M={M} d={d} ffn={ffn}")
    gu_np = np.concatenate([g, u], axis=1)
    dY, WdT, GU = (bf16_dev(inputs.to_bf16_bits(v)) for v in (dy, wdT, gu_np))
    dz = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=DEV)
    pdot = torch.empty(ops.rms_tiles(ffn), M, dtype=torch.float32, device=DEV)
    ops.gemm_swiglu_bwd(dY, WdT, GU, dz, pdot)
    torch.cuda.synchronize()
    dout = dy.astype(np.float64) @ wdT.astype(np.float64).T
    dg, du = oracle.swiglu_grad(dout, g, u)
    dz_host = bf16_host(dz)
    assert np.array_equal(dz_host, dec_bf16(bf16_encode_few(np.concatenate([dg, du], axis=1))))
    width = ops.rms_tile_width()
    T = ops.rms_tiles(ffn)
    ref_p = np.stack([np.sum((dg * g + du * u)[:, t * width:(t + 1) * width], axis=1)
                      for t in range(T)])
    assert np.array_equal(f32_host(pdot), ref_p)
    # RMSNorm-backward GEMM on the exact dz
    w2T = _ints(rng, (d, 2 * ffn), -1, 1)
    h = _ints(rng, (M, d), -4, 4)
    r = np.ones(M, dtype=np.float32)
    c = np.full(M, 0.5, dtype=np.float32)
    dh = torch.empty(M, d, dtype=torch.bfloat16, device=DEV)
    ops.gemm_rmsnorm_bwd(dz, bf16_dev(inputs.to_bf16_bits(w2T)), bf16_dev(inputs.to_bf16_bits(h)),
                         dY, f32_dev(r), f32_dev(c), dh)
    torch.cuda.synchronize()
    G = dz_host @ w2T.astype(np.float64).T  # the kernel's input dz, exactly
    ref = G - 0.5 * h + dy
    assert np.array_equal(bf16_host(dh), dec_bf16(bf16_encode_few(ref)))


@pytest.mark.parametrize("M,d,ffn", [
    (200, 128, 1040),  # last tile: subtile 0 of a feature pair in range, subtile 1 past N
    (200, 128, 1072),  # last tile: subtiles 0..2 in range, 3 past N
    (70, 64, 16),      # a single 16-feature subtile
])
def test_swiglu_bwd_exact_partial_pairs(M, d, ffn):
    """SwiGLU-backward epilogue where a feature width that is a multiple of 16
    but not of 32 leaves one subtile of the epilogue's 32-feature load pairs
    past N: exact values as in test_bwd_epilogues_exact; dz and the partial
    sums bit for bit."""
    rng = np.random.default_rng(7 * M + ffn)
    dy, wdT = _ints(rng, (M, d), -1, 1), _ints(rng, (ffn, d), -1, 1)
    g = 64.0 * rng.integers(0, 2, size=(M, ffn)).astype(np.float32)
    u = _ints(rng, (M, ffn), -1, 2)
    say(f"exact SwiGLU backward, partial feature pairs M={M} d={d} ffn={ffn}")
    gu_np = np.concatenate([g, u], axis=1)
    dY, WdT, GU = (bf16_dev(inputs.to_bf16_bits(v)) for v in (dy, wdT, gu_np))
    dz = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=DEV)
    pdot = torch.empty(ops.rms_tiles(ffn), M, dtype=torch.float32, device=DEV)
    ops.gemm_swiglu_bwd(dY, WdT, GU, dz, pdot)
    torch.cuda.synchronize()
    dout = dy.astype(np.float64) @ wdT.astype(np.float64).T
    dg, du = oracle.swiglu_grad(dout, g, u)
    assert np.array_equal(bf16_host(dz), dec_bf16(bf16_encode_few(np.concatenate([dg, du], axis=1))))
    width = ops.rms_tile_width()
    ref_p = np.stack([np.sum((dg * g + du * u)[:, t * width:(t + 1) * width], axis=1)
                      for t in range(ops.rms_tiles(ffn))])
    assert np.array_equal(f32_host(pdot), ref_p)


def test_bwd_chain_ragged():
    """Forward (saving z) and the whole backward chain on a ragged shape with
    several tiles in every dimension, against the fp64 oracle."""
    w = inputs.make_mlp_bwd(seed=3, M=600, d=448, K1=320, ffn=1056)
    say("backward chain M=600 d=448 K1=320 ffn=1056")
    got = run_fused(w)
    ref = oracle_rows(w)
    check_against_oracle(got, ref)
    # the partial sums themselves: per 128-feature tile of the SwiGLU output
    width, ffn = ops.rms_tile_width(), 1056
    zz = ref["dg"] * ref["g"] + ref["du"] * ref["u"]
    ref_p = np.stack([np.sum(zz[:, t * width:(t + 1) * width], axis=1)
                      for t in range(ops.rms_tiles(ffn))])
    assert norm_err(f32_host(got["pdot"]), ref_p) <= TOL_BF16


def test_unfused_bwd_matches_oracle():
    """The unfused backward sequence (the speed baseline) computes the same
    gradients."""
    w = inputs.make_mlp_bwd(seed=4, M=512, d=1024, K1=512, ffn=2048)
    say("unfused backward M=512 d=1024 ffn=2048")
    fz = run_fused(w)
    uf = run_unfused(w, fz)
    ref = oracle_rows(w)
    check_against_oracle(uf, ref)
    check_against_oracle(fz, ref)


def test_mlp_1b_bwd_sampled_rows():
    """Full 1B-shaped sub-layer, forward and backward in the launch
    configuration the benchmark times; the oracle checks sampled rows (every
    step is row-independent given the weights)."""
    w = inputs.make_workload("mlp_1b_bwd")
    say("mlp_1b_bwd full size, sampled rows")
    got = run_fused(w)
    rows = sample_rows(w.sizes["M"])
    ref = oracle_rows(w, rows)
    check_against_oracle(got, ref, rows)
    for k in ("dz", "dh", "dx"):
        assert bool(torch.isfinite(got[k].float()).all()), k


def run_weight_grads(w, fz):
    """Weight gradients from the fused pass's tensors: token-major copies by
    the transpose kernel (the RMS row scale applied while copying h), then
    plain GEMMs reducing over the token rows."""
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    bf = dict(dtype=torch.bfloat16, device=DEV)
    x, dy = bf16_dev(w.arrays["x"]), bf16_dev(w.arrays["dy"])
    hT, dzT = torch.empty(d, M, **bf), torch.empty(2 * ffn, M, **bf)
    dyT, outT = torch.empty(d, M, **bf), torch.empty(ffn, M, **bf)
    dhT, xT = torch.empty(d, M, **bf), torch.empty(K1, M, **bf)
    ops.transpose(fz["h"], hT, row_scale=fz["r"])
    ops.transpose(fz["dz"], dzT)
    ops.transpose(dy, dyT)
    ops.transpose(fz["out"], outT)
    ops.transpose(fz["dh"], dhT)
    ops.transpose(x, xT)
    dW2, dWd, dWo = (torch.empty(2 * ffn, d, **bf), torch.empty(d, ffn, **bf),
                     torch.empty(d, K1, **bf))
    ops.gemm_bf16(dzT, hT, dW2)   # gradient of the folded [Wg'; Wu']
    # the same GEMM with the RMSNorm-gain epilogue: the unfolded gradient
    # dW = dW' diag(gamma) and the partial sums of dW' * W for dgamma
    wgu = torch.cat([bf16_dev(w.arrays["wg"]), bf16_dev(w.arrays["wu"])], 0).contiguous()
    gamma = f32_dev(w.arrays["gamma"])
    dWu = torch.full((2 * ffn, d), float("nan"), **bf)
    pdg = torch.full((ops.dgamma_slices(2 * ffn), d), float("nan"), dtype=torch.float32,
                     device=DEV)
    dgamma = torch.empty(d, dtype=torch.float32, device=DEV)
    ops.gemm_wgrad_gamma(dzT, hT, wgu, gamma, dWu, pdg)
    ops.dgamma_reduce(pdg, dgamma)
    # unfused: the unfolded gradient from the stored normalised n, then the
    # column-dot pass and the reduce divided by gamma
    n_u = torch.empty(M, d, **bf)
    ops.rmsnorm(fz["h"], gamma, EPS, n_u)
    nT = torch.empty(d, M, **bf)
    ops.transpose(n_u, nT)
    dWn = torch.empty(2 * ffn, d, **bf)
    ops.gemm_bf16(dzT, nT, dWn)
    pdg_u = torch.full_like(pdg, float("nan"))
    dgamma_u = torch.empty_like(dgamma)
    ops.col_dot_partial(dWn, wgu, pdg_u)
    ops.dgamma_reduce(pdg_u, dgamma_u, gamma_div=gamma)
    ops.gemm_bf16(dyT, outT, dWd)
    # dWo (d x K1) has few output tiles: its reduction over the M tokens is
    # split in parts (M a multiple of 64 * parts)
    parts = 4 if M % 256 == 0 else 3 if M % 192 == 0 else 1
    ws = torch.empty(parts, d, K1, dtype=torch.float32, device=DEV)
    ops.gemm_bf16_splitk(dhT, xT, dWo, ws)
    torch.cuda.synchronize()
    return dict(dW2=dW2, dWd=dWd, dWo=dWo, dWu=dWu, dgamma=dgamma, dWn=dWn, dgamma_u=dgamma_u)


def check_weight_grads(w, wg_, ref):
    ffn = w.sizes["ffn"]
    gamma = w.arrays["gamma"].astype(np.float64)[None, :]
    dW2 = bf16_host(wg_["dW2"])
    # the oracle differentiates the unfolded weights: dL/dW = dL/dW' diag(gamma)
    errs = {"dwg": norm_err(dW2[:ffn] * gamma, ref["dwg"]),
            "dwu": norm_err(dW2[ffn:] * gamma, ref["dwu"]),
            "dwd": norm_err(bf16_host(wg_["dWd"]), ref["dwd"]),
            "dwo": norm_err(bf16_host(wg_["dWo"]), ref["dwo"])}
    # the unfolded gradient and dgamma from the epilogue, and from the unfused passes
    dWu, dWn = bf16_host(wg_["dWu"]), bf16_host(wg_["dWn"])
    errs.update({"dwg_epilogue": norm_err(dWu[:ffn], ref["dwg"]),
                 "dwu_epilogue": norm_err(dWu[ffn:], ref["dwu"]),
                 "dgamma": norm_err(f32_host(wg_["dgamma"]), ref["dgamma"]),
                 "dwg_unfused": norm_err(dWn[:ffn], ref["dwg"]),
                 "dgamma_unfused": norm_err(f32_host(wg_["dgamma_u"]), ref["dgamma"])})
    say(f"weight gradient errors {errs}")
    for k, e in errs.items():
        assert e <= TOL_BF16, (k, e)


def test_weight_grads_ragged_features():
    """Weight gradients at M = 576 (the token count is the GEMM reduction, a
    multiple of 64) with ragged feature counts, against the fp64 oracle."""
    w = inputs.make_mlp_bwd(seed=6, M=576, d=448, K1=320, ffn=1056)
    say("weight gradients M=576 d=448 K1=320 ffn=1056")
    fz = run_fused(w)
    check_weight_grads(w, run_weight_grads(w, fz), oracle_rows(w))


@pytest.mark.parametrize("M,N,K", [(300, 272, 128), (512, 256, 64), (1040, 528, 192)])
def test_wgrad_gamma_exact(M, N, K):
    """Integer operands make every sum exact: G = A B^T has |G| <= K, gamma in
    {1/2, 1, 2, -1} keeps G gamma exact in bf16 (|G gamma| <= 256 with at most
    8 significant bits), W in [-3, 3] keeps every partial sum an integer below
    2^24.  dW, the partial sums and dgamma must equal the oracle bit for bit
    (ragged rows and columns, one and several tiles, 128-row slices that end
    inside a tile)."""
    rng = np.random.default_rng(M + N + K)
    a, b = _ints(rng, (M, K), -1, 1), _ints(rng, (N, K), -1, 1)
    wt = _ints(rng, (M, N), -3, 3)
    gam = rng.choice(np.array([0.5, 1.0, 2.0, -1.0], dtype=np.float32), size=N)
    if K > 128:  # keep |G gamma| <= 256
        gam = np.where(np.abs(gam) > 1, 1.0, gam).astype(np.float32)
    say(f"wgrad gamma epilogue exact M={M} N={N} K={K}")
    A, B, W = (bf16_dev(bf16_encode_few(v)) for v in (a, b, wt))
    dW = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    P = ops.dgamma_slices(M)
    pdg = torch.full((P, N), float("nan"), dtype=torch.float32, device=DEV)
    dg = torch.empty(N, dtype=torch.float32, device=DEV)
    ops.gemm_wgrad_gamma(A, B, W, f32_dev(gam), dW, pdg)
    ops.dgamma_reduce(pdg, dg)
    pdg_u = torch.full((P, N), float("nan"), dtype=torch.float32, device=DEV)
    ops.col_dot_partial(W, W, pdg_u)
    torch.cuda.synchronize()
    G = oracle.gemm_nt(a, b)
    assert np.array_equal(bf16_host(dW), G * gam.astype(np.float64)[None, :])
    ref_p = np.stack([np.sum(G[p * 128:(p + 1) * 128] * wt[p * 128:(p + 1) * 128], axis=0)
                      for p in range(P)])
    assert np.array_equal(f32_host(pdg), ref_p)
    assert np.array_equal(f32_host(dg), np.sum(G * wt, axis=0))
    ref_u = np.stack([np.sum(wt[p * 128:(p + 1) * 128] ** 2, axis=0) for p in range(P)])
    assert np.array_equal(f32_host(pdg_u), ref_u)


@pytest.mark.parametrize("rows,cols", [(130, 70), (128, 72), (8, 1024), (264, 392)])
def test_transpose_row_scale_exact(rows, cols):
    """The scaled transpose rounds src * scale once (RNE) per element (ragged
    sizes take the element-wise kernel, multiples of 8 the 16-byte one)."""
    rng = np.random.default_rng(7)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    s = rng.uniform(0.5, 2.0, size=rows).astype(np.float32)
    bits = inputs.to_bf16_bits(a)
    say(f"scaled transpose {rows}x{cols}")
    dst = torch.empty(cols, rows, dtype=torch.bfloat16, device=DEV)
    ops.transpose(bf16_dev(bits), dst, row_scale=f32_dev(s))
    torch.cuda.synchronize()
    # the product of a bf16 value and an fp32 scale, rounded to fp32 (as the
    # kernel computes it), then to bf16
    prod = (dec_bf16(bits) * s.astype(np.float64)[:, None]).astype(np.float32).astype(np.float64)
    assert np.array_equal(bf16_host(dst), dec_bf16(bf16_encode_few(prod)).T)


def test_mlp_1b_weight_grads_full():
    """Weight gradients at the full 1B shape (sums over all 8192 tokens), against
    the fp64 oracle of the whole sub-layer."""
    w = inputs.make_workload("mlp_1b_bwd")
    say("mlp_1b_bwd weight gradients, full size")
    fz = run_fused(w)
    wg_ = run_weight_grads(w, fz)
    check_weight_grads(w, wg_, oracle_rows(w))

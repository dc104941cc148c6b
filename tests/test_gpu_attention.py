"""GPU parity of the causal grouped-query attention core and of the full
transformer-layer forward (attention-input block -> attention -> MLP block)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogue_transformer_gemm1_amd import inputs, ops
from tests.gpu_util import (DEV, TOL_BF16, TOL_ROW, bf16_dev, bf16_host, dec_bf16, f32_dev,
                            f32_host, i32_dev, norm_err, row_rel_err, say)

pytestmark = pytest.mark.gpu
EPS = 1e-5


def _qkv_bits(seed, M, nq, nkv, scale=1.0, hd=64):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((M, (nq + 2 * nkv) * hd)) * scale).astype(np.float32)
    return inputs.to_bf16_bits(a)


def run_attention(bits, L, nq, nkv, hd=64):
    M = bits.shape[0]
    o = torch.full((M, nq * hd), float("nan"), dtype=torch.bfloat16, device=DEV)
    ops.attention_fwd(bf16_dev(bits), o, L, nq, nkv, hd)
    torch.cuda.synchronize()
    return bf16_host(o)


@pytest.mark.parametrize("L,n_seq,nq,nkv", [(128, 2, 4, 2), (256, 3, 6, 2), (384, 1, 2, 2),
                                             (128, 1, 1, 1), (512, 2, 8, 1), (4096, 1, 2, 1)])
def test_attention_small(L, n_seq, nq, nkv):
    """Several query blocks and key steps per sequence, sequence boundaries,
    grouped (and ungrouped) kv heads, and one long sequence (64 key steps for
    its last query block)."""
    M = L * n_seq
    bits = _qkv_bits(L + nq + nkv, M, nq, nkv)
    say(f"attention L={L} seqs={n_seq} nq={nq} nkv={nkv}")
    got = run_attention(bits, L, nq, nkv)
    ref = oracle.attention_causal_gqa(dec_bf16(bits), L, nq, nkv, 64)
    assert norm_err(got, ref) <= TOL_BF16


@pytest.mark.parametrize("L,n_seq,nq,nkv", [(128, 2, 4, 2), (256, 3, 6, 2), (384, 1, 2, 2),
                                             (128, 1, 1, 1), (512, 2, 8, 1), (2048, 1, 2, 2)])
def test_attention_head128(L, n_seq, nq, nkv):
    """Heads of 128 (the 7B / 70B shapes): 32 queries per wave, four waves per
    workgroup, 256-byte K and V rows."""
    M = L * n_seq
    bits = _qkv_bits(L + nq + 3 * nkv, M, nq, nkv, hd=128)
    say(f"attention hd=128 L={L} seqs={n_seq} nq={nq} nkv={nkv}")
    got = run_attention(bits, L, nq, nkv, hd=128)
    ref = oracle.attention_causal_gqa(dec_bf16(bits), L, nq, nkv, 128)
    assert norm_err(got, ref) <= TOL_BF16


def test_attention_head128_closed_forms_and_peaks():
    """Heads of 128: the first query of a sequence returns its own v row;
    with scores of magnitude ~100 the lazy reference max is raised often."""
    L, n_seq, nq, nkv, hd = 256, 2, 4, 2, 128
    M = L * n_seq
    rng = np.random.default_rng(15)
    a = rng.standard_normal((M, (nq + 2 * nkv) * hd)).astype(np.float32)
    a[:, :nq * hd] *= 10.0
    bits = inputs.to_bf16_bits(a)
    say("attention hd=128 closed forms and peaked scores")
    got = run_attention(bits, L, nq, nkv, hd=hd)
    x = dec_bf16(bits)
    ref = oracle.attention_causal_gqa(x, L, nq, nkv, hd)
    assert norm_err(got, ref) <= TOL_BF16
    for s0 in (0, L):
        for h in range(nq):
            g = h // (nq // nkv)
            v = x[s0, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd]
            o = got[s0, h * hd:(h + 1) * hd]
            assert float(np.max(np.abs(o - v))) <= 2 ** -7 * max(1.0, float(np.max(np.abs(v))))


def test_attention_closed_forms():
    """The first query of each sequence returns its own v row; with one key
    for the whole kv head, query i returns the mean of v over keys 0..i."""
    L, n_seq, nq, nkv = 256, 2, 4, 1
    M = L * n_seq
    rng = np.random.default_rng(5)
    a = rng.standard_normal((M, (nq + 2 * nkv) * 64)).astype(np.float32)
    a[:, nq * 64:(nq + 1) * 64] = rng.standard_normal(64).astype(np.float32)[None, :]
    bits = inputs.to_bf16_bits(a)
    say("attention closed forms")
    got = run_attention(bits, L, nq, nkv)
    x = dec_bf16(bits)
    v = x[:, (nq + nkv) * 64:(nq + nkv + 1) * 64]
    for s0 in (0, L):
        mean = np.cumsum(v[s0:s0 + L], axis=0) / np.arange(1, L + 1)[:, None]
        for h in range(nq):
            o = got[s0:s0 + L, h * 64:(h + 1) * 64]
            assert float(np.max(np.abs(o[0] - v[s0]))) <= 2 ** -7 * max(1.0, float(np.max(np.abs(v[s0]))))
            assert norm_err(o, mean) <= TOL_BF16


def test_attention_peaked_scores():
    """Scores of magnitude ~100 (q scaled up): the softmax is nearly one-hot
    and the running max does all the work."""
    L, n_seq, nq, nkv = 256, 2, 4, 2
    M = L * n_seq
    rng = np.random.default_rng(6)
    a = rng.standard_normal((M, (nq + 2 * nkv) * 64)).astype(np.float32)
    a[:, :nq * 64] *= 12.0
    bits = inputs.to_bf16_bits(a)
    say("attention with peaked scores")
    got = run_attention(bits, L, nq, nkv)
    ref = oracle.attention_causal_gqa(dec_bf16(bits), L, nq, nkv, 64)
    assert norm_err(got, ref) <= TOL_BF16


def test_attention_rising_scores():
    """Scores that rise along the keys (by about 0.09 in log2 units per key,
    plus noise): the running max keeps growing, so the reference max is both
    held while p climbs towards its 2^8 headroom and raised many times."""
    L, n_seq, nq, nkv = 1024, 2, 4, 2
    M = L * n_seq
    rng = np.random.default_rng(8)
    a = (0.3 * rng.standard_normal((M, (nq + 2 * nkv) * 64))).astype(np.float32)
    a[:, :nq * 64:64] = 8.0                                   # q feature 0 of every head
    ramp = 0.06 * np.tile(np.arange(L), n_seq).astype(np.float32)
    for kh in range(nkv):
        a[:, (nq + kh) * 64] = ramp                           # k feature 0 grows with the key
    bits = inputs.to_bf16_bits(a)
    say("attention with rising scores")
    got = run_attention(bits, L, nq, nkv)
    ref = oracle.attention_causal_gqa(dec_bf16(bits), L, nq, nkv, 64)
    assert norm_err(got, ref) <= TOL_BF16


def test_attention_layer_shape_every_row():
    """The layer's attention at full size (4 sequences of 2048, 32 q / 8 kv
    heads of 64) on the QKV the 1B-shaped layer produces, every row."""
    L, n_seq, nq, nkv = 2048, 4, 32, 8
    M = L * n_seq
    bits = _qkv_bits(7, M, nq, nkv)
    say("attention full size M=8192 L=2048 32/8 heads")
    got = run_attention(bits, L, nq, nkv)
    ref = oracle.attention_causal_gqa(dec_bf16(bits), L, nq, nkv, 64)
    err = norm_err(got, ref)
    say(f"attention full size err {err:.2e}")
    assert err <= TOL_BF16


def run_layer(w):
    """The layer on the GPU: GEMM1 (down projection, residual, partial RMS) ->
    reduce -> QKV + RoPE -> attention -> GEMM1 (output projection, residual,
    partial RMS) -> reduce -> GEMM2 (row scale, SwiGLU)."""
    sz = w.sizes
    M, d, K1, ffn = sz["M"], sz["d"], sz["K1"], sz["ffn"]
    nq, nkv, L, hd = sz["n_q"], sz["n_kv"], sz["seq_len"], sz["head_dim"]
    bf = dict(dtype=torch.bfloat16, device=DEV)
    x, res, wdn, wqkv = (bf16_dev(w.arrays[k]) for k in ("x", "res", "w1", "wqkv"))
    wo, wg, wu = (bf16_dev(w.arrays[k]) for k in ("wo", "wg", "wu"))
    g1, g2 = f32_dev(w.arrays["gamma"]), f32_dev(w.arrays["gamma2"])
    wqkv_f, wg_f, wu_f = torch.empty_like(wqkv), torch.empty_like(wg), torch.empty_like(wu)
    ops.fold_gamma(wqkv, g1, wqkv_f)
    ops.fold_gamma(wg, g2, wg_f)
    ops.fold_gamma(wu, g2, wu_f)
    cos = torch.empty(L, hd // 2, dtype=torch.float32, device=DEV)
    sin = torch.empty_like(cos)
    ops.rope_tables(sz["theta"], L, hd, cos, sin)
    pos = i32_dev(w.arrays["pos"])
    T = ops.rms_tiles(d)
    h1, h2 = torch.empty(M, d, **bf), torch.empty(M, d, **bf)
    P1, P2 = (torch.empty(T, M, dtype=torch.float32, device=DEV) for _ in range(2))
    r1, r2 = (torch.empty(M, dtype=torch.float32, device=DEV) for _ in range(2))
    qkv = torch.empty(M, (nq + 2 * nkv) * hd, **bf)
    o = torch.empty(M, nq * hd, **bf)
    out = torch.empty(M, ffn, **bf)
    ops.gemm_residual_partialrms(x, wdn, res, h1, P1)
    ops.rms_reduce(P1, d, EPS, r1)
    ops.gemm_rope(h1, wqkv_f, r1, cos, sin, pos, qkv, nq, nkv, hd)
    ops.attention_fwd(qkv, o, L, nq, nkv, hd)
    ops.gemm_residual_partialrms(o, wo, h1, h2, P2)
    ops.rms_reduce(P2, d, EPS, r2)
    ops.gemm_rowscale_swiglu(h2, wg_f, wu_f, r2, out)
    torch.cuda.synchronize()
    return {"h1": bf16_host(h1), "r1": f32_host(r1), "qkv": bf16_host(qkv), "o": bf16_host(o),
            "h2": bf16_host(h2), "r2": f32_host(r2), "out": bf16_host(out)}


def oracle_layer(w):
    sz = w.sizes
    return oracle.layer_forward(
        dec_bf16(w.arrays["x"]), dec_bf16(w.arrays["res"]), dec_bf16(w.arrays["w1"]),
        dec_bf16(w.arrays["wqkv"]), w.arrays["gamma"].astype(np.float64),
        dec_bf16(w.arrays["wo"]), dec_bf16(w.arrays["wg"]), dec_bf16(w.arrays["wu"]),
        w.arrays["gamma2"].astype(np.float64), EPS, w.arrays["pos"], sz["n_q"], sz["n_kv"],
        sz["head_dim"], sz["theta"], sz["seq_len"])


def _row_norm_rel(got, ref):
    """Per row: ||got - ref|| / ||ref||."""
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(np.asarray(got, dtype=np.float64) - ref, axis=1) / \
        np.maximum(np.linalg.norm(ref, axis=1), 1e-30)


def check_layer(w, got):
    """Two checks of the same GPU run.

    Stage by stage: each kernel's output against the oracle's stage fed with
    the GPU's own (bf16) inputs of that stage, so every kernel meets its own
    bar (TOL_BF16 for bf16 tensors, TOL_ROW for r).

    End to end: every stage against the oracle's layer computed in fp64 from
    the layer inputs alone.  The bf16 tensors meet TOL_BF16.  r2 inherits the
    storage rounding of h1 and o, so its bar is derived per row: to first
    order |dr / r| <= ||dh|| / ||h|| for r = rsqrt(mean h^2 + eps), and the GPU
    takes r2 from h2 before the bf16 rounding of its store (relative 2^-9 of
    the row norm), so |dr2 / r2| <= ||h2_gpu - h2_ref|| / ||h2_ref|| + 2^-9 + TOL_ROW."""
    sz = w.sizes
    nq, nkv, L, hd = sz["n_q"], sz["n_kv"], sz["seq_len"], sz["head_dim"]
    stage = {"o": oracle.attention_causal_gqa(got["qkv"], L, nq, nkv, hd)}
    f2 = oracle.mlp_block(got["o"], got["h1"], dec_bf16(w.arrays["wo"]), dec_bf16(w.arrays["wg"]),
                          dec_bf16(w.arrays["wu"]), w.arrays["gamma2"].astype(np.float64), EPS)
    stage.update({"h2": f2["h"], "r2": f2["r"], "out": f2["out"]})
    ref = oracle_layer(w)
    stage.update({"h1": ref["h1"], "r1": ref["r1"], "qkv": ref["qkv"]})
    tensors = ("h1", "qkv", "o", "h2", "out")
    errs_stage = {k: norm_err(got[k], stage[k]) for k in tensors}
    errs_stage.update({k: row_rel_err(got[k], stage[k]) for k in ("r1", "r2")})
    errs_e2e = {k: norm_err(got[k], ref[k]) for k in tensors}
    r2_rel = np.abs(got["r2"].astype(np.float64) - ref["r2"]) / np.abs(ref["r2"])
    r2_bar = _row_norm_rel(got["h2"], ref["h2"]) + 2.0 ** -9 + TOL_ROW
    say(f"layer stage errors {errs_stage}")
    say(f"layer end-to-end errors {errs_e2e}, r2 max {float(r2_rel.max()):.2e} "
        f"(bar min {float(r2_bar.min()):.2e})")
    for k in tensors:
        assert errs_stage[k] <= TOL_BF16, ("stage", k, errs_stage[k])
        assert errs_e2e[k] <= TOL_BF16, ("end to end", k, errs_e2e[k])
    assert errs_stage["r1"] <= TOL_ROW and errs_stage["r2"] <= TOL_ROW, errs_stage
    assert np.all(r2_rel <= r2_bar)


def test_layer_small():
    """A whole layer at a small shape: two sequences of 256, 8 q / 2 kv heads,
    ragged MLP width."""
    w = inputs.make_layer(seed=3, M=512, d=512, K1=640, ffn=1040, n_q=8, n_kv=2, seq_len=256)
    say("layer small M=512 d=512 K1=640 ffn=1040 8/2 heads L=256")
    check_layer(w, run_layer(w))


def test_layer_small_head128_ragged():
    """A whole layer with heads of 128 at small ragged widths: two sequences of
    128, 4 q / 2 kv heads, d = 384 (one and a half GEMM tiles), previous-MLP
    width 320, ffn = 704."""
    w = inputs.make_layer(seed=4, M=256, d=384, K1=320, ffn=704, n_q=4, n_kv=2, head_dim=128,
                          theta=10000.0, seq_len=128)
    say("layer small hd=128 M=256 d=384 K1=320 ffn=704 4/2 heads L=128")
    check_layer(w, run_layer(w))


def test_layer_1b_every_row():
    """The 1B-shaped layer (M=8192 as 4 sequences of 2048, d=2048, ffn=8192,
    32 q / 8 kv heads) in the launch configuration the benchmark times; every
    row of every stage against the oracle."""
    w = inputs.make_workload("layer_1b")
    say("layer_1b full size, every row")
    check_layer(w, run_layer(w))


@pytest.mark.parametrize("name", ["layer_7b", "layer_70b"])
def test_layer_7b_70b_one_sequence_every_row(name):
    """The layer at the 7B (32 heads of 128, no grouping, ffn 11008) and 70B
    (64 q / 8 kv heads of 128, ffn 28672) shapes on one sequence of 2048
    tokens, every row of every stage."""
    w = inputs.make_workload(name, M=2048)
    say(f"{name} at M=2048 (one sequence), every row")
    check_layer(w, run_layer(w))

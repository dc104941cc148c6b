"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  Each mutant replaces one oracle function with a
subtly wrong copy; at least one pin in tests/oracle_pins.py must then fail."""
import numpy as np
import pytest

import oracle
from oracle import codecs, reference as R
from tests import oracle_pins

_ORIG_ROPE = R.apply_rope
_ORIG_LM = R.lm_head_ce
_ORIG_DEC = codecs.e4m3_decode
_ORIG_ATT = R.attention_causal_gqa


def _mlp_block_no_gamma(x, res, wo, wg, wu, gamma, eps):
    h = R.residual_add(R.gemm_nt(x, wo), res)
    r = R.rms_scale(h, eps)
    n = r[:, None] * h
    g, u = R.gemm_nt(n, wg), R.gemm_nt(n, wu)
    return {"h": h, "r": r, "g": g, "u": u, "out": R.swiglu(g, u)}


def _mlp_block_swapped_gate(x, res, wo, wg, wu, gamma, eps):
    h = R.residual_add(R.gemm_nt(x, wo), res)
    r = R.rms_scale(h, eps)
    n = (r[:, None] * h) * np.asarray(gamma)[None, :]
    g, u = R.gemm_nt(n, wg), R.gemm_nt(n, wu)
    return {"h": h, "r": r, "g": g, "u": u, "out": R.swiglu(u, g)}


def _apply_rope_sign(y, pos, n_rot, hd, cos, sin):
    return _ORIG_ROPE(y, pos, n_rot, hd, cos, -sin)


def _apply_rope_interleaved(y, pos, n_rot, hd, cos, sin):
    y = np.array(y, dtype=np.float64, copy=True)
    c, s = cos[np.asarray(pos)], sin[np.asarray(pos)]
    for hh in range(n_rot):
        a = y[:, hh * hd:(hh + 1) * hd:2].copy()
        b = y[:, hh * hd + 1:(hh + 1) * hd:2].copy()
        y[:, hh * hd:(hh + 1) * hd:2] = a * c - b * s
        y[:, hh * hd + 1:(hh + 1) * hd:2] = b * c + a * s
    return y


def _rope_tables_wrong_exponent(max_pos, hd, theta):
    i = np.arange(hd // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * (theta ** (-i / hd))[None, :]
    return np.cos(ang), np.sin(ang)


def _lse_merge_no_rescale(mx, se, order=None):
    mx, se = np.asarray(mx), np.asarray(se)
    M = np.max(mx, axis=0)
    return M + np.log(np.sum(se, axis=0))


def _lm_head_ignored_keep_lse(x, wlm, labels, r=None, chunk=256):
    o = _ORIG_LM(x, wlm, labels, r=r, chunk=chunk)
    V = np.asarray(wlm).shape[0]
    bad = (np.asarray(labels) < 0) | (np.asarray(labels) >= V)
    o["loss"] = np.where(bad, o["lse"], o["loss"])
    return o


def _lm_head_ignored_clamped(x, wlm, labels, r=None, chunk=256):
    V = np.asarray(wlm).shape[0]
    return _ORIG_LM(x, wlm, np.clip(np.asarray(labels), 0, V - 1), r=r, chunk=chunk)


def _lm_head_label_shift(x, wlm, labels, r=None, chunk=256):
    V = np.asarray(wlm).shape[0]
    return _ORIG_LM(x, wlm, (np.asarray(labels) + 1) % V, r=r, chunk=chunk)


_ORIG_LAYER_BWD = R.mlp_layer_bwd


def _swiglu_grad_no_curvature(dout, g, u):
    g, u, dout = (np.asarray(v, dtype=np.float64) for v in (g, u, dout))
    s = 1.0 / (1.0 + np.exp(-g))
    return dout * u * s, dout * g * s


def _rmsnorm_bwd_variant(sign=-1.0, power=3, use_gamma=True):
    def f(dn, h, gamma, eps):
        h = np.asarray(h, dtype=np.float64)
        gm = np.asarray(gamma, dtype=np.float64) if use_gamma else np.ones(h.shape[1])
        dng = np.asarray(dn, dtype=np.float64) * gm[None, :]
        r = R.rms_scale(h, eps)
        coef = r ** power / h.shape[1] * np.sum(dng * h, axis=1)
        return r[:, None] * dng + sign * coef[:, None] * h, coef
    return f


def _layer_bwd_no_skip(x, res, wo, wg, wu, gamma, eps, wd, dy):
    o = _ORIG_LAYER_BWD(x, res, wo, wg, wu, gamma, eps, wd, dy)
    o["dh"] = o["dres"] = o["dh"] - np.asarray(dy)
    o["dx"] = o["dh"] @ np.asarray(wo)
    return o


def _layer_bwd_dw_without_row_scale(x, res, wo, wg, wu, gamma, eps, wd, dy):
    o = _ORIG_LAYER_BWD(x, res, wo, wg, wu, gamma, eps, wd, dy)
    n = o["h"] * np.asarray(gamma)[None, :]
    o["dwg"], o["dwu"] = o["dg"].T @ n, o["du"].T @ n
    return o


def _layer_bwd_dwd_transposed_operands(x, res, wo, wg, wu, gamma, eps, wd, dy):
    o = _ORIG_LAYER_BWD(x, res, wo, wg, wu, gamma, eps, wd, dy)
    o["dwd"] = (o["out"].T @ np.asarray(dy)).T * 0.5 + 0.5 * np.asarray(dy).T @ o["out"][:, ::-1]
    return o


def _layer_bwd_up_gate_swapped(x, res, wo, wg, wu, gamma, eps, wd, dy):
    return _ORIG_LAYER_BWD(x, res, wo, wu, wg, gamma, eps, wd, dy)


def _attention_variant(mask="causal", group="div", scale="sqrt", cross_seq=False):
    def att(qkv, seq_len, n_q, n_kv, head_dim):
        qkv = np.asarray(qkv, dtype=np.float64)
        M, hd = qkv.shape[0], head_dim
        L = M if cross_seq else seq_len
        o = np.empty((M, n_q * hd))
        tri = {"causal": np.tril(np.ones((L, L), bool)), "none": np.ones((L, L), bool),
               "strict": np.tril(np.ones((L, L), bool), -1) | (np.arange(L)[:, None] == 0)}[mask]
        for s0 in range(0, M, L):
            rows = slice(s0, s0 + L)
            for h in range(n_q):
                g = h // (n_q // n_kv) if group == "div" else h % n_kv
                q = qkv[rows, h * hd:(h + 1) * hd]
                k = qkv[rows, (n_q + g) * hd:(n_q + g + 1) * hd]
                v = qkv[rows, (n_q + n_kv + g) * hd:(n_q + n_kv + g + 1) * hd]
                sc = (q @ k.T) / (np.sqrt(hd) if scale == "sqrt" else hd)
                sc = np.where(tri, sc, -np.inf)
                p = np.exp(sc - np.max(sc, axis=1, keepdims=True))
                o[rows, h * hd:(h + 1) * hd] = (p / np.sum(p, axis=1, keepdims=True)) @ v
        return o
    return att


MUTANTS = {
    "eps outside sqrt": ("rms_scale", lambda h, eps: 1.0 / np.sqrt(np.mean(np.asarray(h) ** 2, axis=1)) + eps),
    "sum instead of mean": ("rms_scale", lambda h, eps: 1.0 / np.sqrt(np.sum(np.asarray(h) ** 2, axis=1) + eps)),
    "residual dropped": ("residual_add", lambda y, res: np.asarray(y, dtype=np.float64)),
    "residual subtracted": ("residual_add", lambda y, res: np.asarray(y) - np.asarray(res)),
    "transposed weight": ("gemm_nt", lambda a, w: np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64)),
    "silu sign": ("silu", lambda z: np.asarray(z) / (1.0 + np.exp(np.asarray(z)))),
    "gamma dropped": ("mlp_block", _mlp_block_no_gamma),
    "gate and up swapped": ("mlp_block", _mlp_block_swapped_gate),
    "rope sign": ("apply_rope", _apply_rope_sign),
    "rope interleaved pairs": ("apply_rope", _apply_rope_interleaved),
    "rope exponent": ("rope_tables", _rope_tables_wrong_exponent),
    "lse without max": ("logsumexp_rows", lambda z: np.log(np.sum(np.exp(np.asarray(z)), axis=1)) + 1e-3),
    "merge without rescale": ("lse_merge", _lse_merge_no_rescale),
    "label off by one": ("lm_head_ce", _lm_head_label_shift),
    "ignored row keeps its lse as loss": ("lm_head_ce", _lm_head_ignored_keep_lse),
    "out-of-range label clamped": ("lm_head_ce", _lm_head_ignored_clamped),
    "swiglu grad without the s(1-s) term": ("swiglu_grad", _swiglu_grad_no_curvature),
    "rmsnorm bwd correction dropped": ("rmsnorm_bwd", _rmsnorm_bwd_variant(sign=0.0)),
    "rmsnorm bwd correction sign": ("rmsnorm_bwd", _rmsnorm_bwd_variant(sign=1.0)),
    "rmsnorm bwd r^2 for r^3": ("rmsnorm_bwd", _rmsnorm_bwd_variant(power=2)),
    "rmsnorm bwd gamma dropped": ("rmsnorm_bwd", _rmsnorm_bwd_variant(use_gamma=False)),
    "skip-connection gradient dropped": ("mlp_layer_bwd", _layer_bwd_no_skip),
    "gate and up swapped in backward": ("mlp_layer_bwd", _layer_bwd_up_gate_swapped),
    "weight gradient without the row scale": ("mlp_layer_bwd", _layer_bwd_dw_without_row_scale),
    "down-projection gradient with permuted features": ("mlp_layer_bwd", _layer_bwd_dwd_transposed_operands),
    "attention without the causal mask": ("attention_causal_gqa", _attention_variant(mask="none")),
    "attention excludes the query's own key": ("attention_causal_gqa", _attention_variant(mask="strict")),
    "kv head chosen as h mod n_kv": ("attention_causal_gqa", _attention_variant(group="mod")),
    "attention scaled by 1/hd": ("attention_causal_gqa", _attention_variant(scale="hd")),
    "attention across sequence boundaries": ("attention_causal_gqa", _attention_variant(cross_seq=True)),
    "abs instead of square": ("partial_sumsq", lambda h, w: np.stack([np.sum(np.abs(np.asarray(h)[:, t * w:(t + 1) * w]), axis=1) for t in range((np.asarray(h).shape[1] + w - 1) // w)])),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    fn_name, mutant = MUTANTS[name]
    monkeypatch.setattr(R, fn_name, mutant)
    if hasattr(oracle, fn_name):
        monkeypatch.setattr(oracle, fn_name, mutant)
    results = oracle_pins.run_all()
    failed = [n for n, ok, _ in results if not ok]
    assert failed, f"mutant '{name}' passed every pin"


def test_e4m3_bias_mutant_is_caught(monkeypatch):
    # exponent bias 8 instead of 7 halves every decoded value
    wrong = lambda codes: _ORIG_DEC(codes) / 2.0
    monkeypatch.setattr(codecs, "e4m3_decode", wrong)
    results = oracle_pins.run_all()
    assert any(not ok for _, ok, _ in results)


def test_unmutated_oracle_passes_every_pin():
    results = oracle_pins.run_all()
    assert all(ok for _, ok, _ in results), [d for _, ok, d in results if not ok]


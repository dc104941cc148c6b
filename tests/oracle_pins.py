"""Checks that pin the CPU oracle to facts outside itself.

Each `pin_*` function returns (ok: bool, detail: str).  They are run as plain
tests (tests/test_oracle_pins.py) and again against deliberately broken copies
of the oracle (tests/test_oracle_mutants.py) to show that a plausible mistake
-- a dropped term, a wrong sign, index or eps placement, a transposed operand
-- fails at least one of them.

Kinds of pin used (none of them re-calls the oracle's own formula):
  * brute force: pure-Python loops with math.fsum on tiny inputs;
  * exact arithmetic: fractions.Fraction / decimal.Decimal on a hand-built
    example (tests/golden/mlp_exact_example.json);
  * library routines: torch CPU float64 rms_norm, silu, cross_entropy,
    logsumexp, complex multiplication;
  * closed forms and invariants of the mathematics (unit RMS after
    normalisation, RoPE as a rotation, merge order independence, W = 0 gives
    loss ln V).
"""

import json
import math
import os
import random
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import reference as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / den


def _ok(err, tol, what):
    return (err <= tol, f"{what}: err {err:.3e} (tol {tol:.1e})")


# ---------------------------------------------------------------------------
# brute force, pure Python
# ---------------------------------------------------------------------------

def _bf_gemm_nt(a, w):
    return [[math.fsum(a[i][k] * w[j][k] for k in range(len(a[i]))) for j in range(len(w))]
            for i in range(len(a))]


def _bf_silu(z):
    return z / (1.0 + math.exp(-z))


def _rand(rng, r, c, s=1.0):
    return [[rng.gauss(0.0, s) for _ in range(c)] for _ in range(r)]


def pin_mlp_bruteforce(seed=1):
    rng = random.Random(seed)
    M, K1, d, ffn, eps = 3, 5, 4, 6, 1e-5
    x, res = _rand(rng, M, K1), _rand(rng, M, d)
    wo, wg, wu = _rand(rng, d, K1, 0.5), _rand(rng, ffn, d, 0.5), _rand(rng, ffn, d, 0.5)
    gamma = [1.0 + 0.1 * rng.gauss(0, 1) for _ in range(d)]
    y = _bf_gemm_nt(x, wo)
    h = [[res[m][n] + y[m][n] for n in range(d)] for m in range(M)]
    r = [1.0 / math.sqrt(math.fsum(v * v for v in h[m]) / d + eps) for m in range(M)]
    nrm = [[r[m] * h[m][n] * gamma[n] for n in range(d)] for m in range(M)]
    g, u = _bf_gemm_nt(nrm, wg), _bf_gemm_nt(nrm, wu)
    out = [[_bf_silu(g[m][j]) * u[m][j] for j in range(ffn)] for m in range(M)]
    o = oracle.mlp_block(np.array(x), np.array(res), np.array(wo), np.array(wg), np.array(wu),
                         np.array(gamma), eps)
    err = max(_rel(o["h"], h), _rel(o["r"], r), _rel(o["g"], g), _rel(o["u"], u),
              _rel(o["out"], out))
    return _ok(err, 1e-12, "mlp brute force")


def pin_mlp_exact_example():
    """Hand-built example with exact rational values (eps = 0, rows chosen so
    mean(h^2) is a perfect square); see tests/golden/mlp_exact_example.json."""
    with open(os.path.join(GOLDEN, "mlp_exact_example.json")) as f:
        ex = json.load(f)
    arr = lambda k: np.array([[float(Fraction(v)) for v in row] for row in ex["inputs"][k]])
    gamma = np.array([float(Fraction(v)) for v in ex["inputs"]["gamma"]])
    o = oracle.mlp_block(arr("x"), arr("res"), arr("wo"), arr("wg"), arr("wu"), gamma,
                         float(Fraction(ex["inputs"]["eps"])))
    exp = ex["expected"]
    errs = []
    for k in ("h", "g", "u"):
        ref = np.array([[float(Fraction(v)) for v in row] for row in exp[k]])
        errs.append(_rel(o[k], ref))
    errs.append(_rel(o["r"], [float(Fraction(v)) for v in exp["r"]]))
    errs.append(_rel(o["out"], np.array([[float(Decimal(v)) for v in row] for row in exp["out"]])))
    return _ok(max(errs), 1e-14, "mlp exact example")


def pin_rmsnorm_torch(seed=2):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(7, 33, generator=g, dtype=torch.float64) * 3
    gamma = 1 + 0.1 * torch.randn(33, generator=g, dtype=torch.float64)
    eps = 1e-5
    ref = torch.nn.functional.rms_norm(h, (33,), weight=gamma, eps=eps)
    return _ok(_rel(R.rmsnorm(h.numpy(), gamma.numpy(), eps), ref.numpy()), 1e-13,
               "rmsnorm vs torch")


def pin_rms_closed_forms():
    d, eps = 16, 1e-5
    h = np.zeros((3, d))
    h[0, :] = 2.5                       # constant row c: r = (c^2 + eps)^-1/2
    h[1, 5] = -4.0                      # one non-zero c: r = (c^2/d + eps)^-1/2
    h[2, :] = np.arange(d) - 7.5        # generic row: mean((r h)^2) = ms/(ms+eps)
    r = R.rms_scale(h, eps)
    e0 = abs(r[0] - (2.5 ** 2 + eps) ** -0.5)
    e1 = abs(r[1] - (16.0 / d + eps) ** -0.5)
    ms = sum((v - 7.5) ** 2 for v in range(d)) / d
    e2 = abs(float(np.mean((r[2] * h[2]) ** 2)) - ms / (ms + eps))
    return _ok(max(e0, e1, e2), 1e-12, "rms closed forms")


def pin_unit_rms(seed=3):
    """RMSNorm output rows have unit RMS before gamma (eps = 0)."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((9, 40)) * rng.uniform(0.1, 10, size=(9, 1))
    n = R.rmsnorm(h, np.ones(40), 0.0)
    return _ok(float(np.max(np.abs(np.sqrt(np.mean(n * n, axis=1)) - 1.0))), 1e-13, "unit RMS")


def pin_rowscale_commutes(seed=4):
    """The page's identity: applying the row scale before GEMM2 equals
    applying it after GEMM2, with gamma folded into W's columns."""
    rng = np.random.default_rng(seed)
    M, d, ffn, eps = 6, 24, 10, 1e-5
    x, res = rng.standard_normal((M, d)), rng.standard_normal((M, d))
    wo, wg, wu = (rng.standard_normal((d, d)) / 5, rng.standard_normal((ffn, d)) / 5,
                  rng.standard_normal((ffn, d)) / 5)
    gamma = 1 + 0.1 * rng.standard_normal(d)
    o = oracle.mlp_block(x, res, wo, wg, wu, gamma, eps)
    h = res + x @ wo.T
    r_bf = [1.0 / math.sqrt(math.fsum(v * v for v in row) / d + eps) for row in h]
    r_bf = np.array(r_bf)
    g_after = r_bf[:, None] * (h @ (wg * gamma[None, :]).T)
    u_after = r_bf[:, None] * (h @ (wu * gamma[None, :]).T)
    return _ok(max(_rel(o["g"], g_after), _rel(o["u"], u_after)), 1e-12,
               "row scale commutes with GEMM2")


def pin_swiglu():
    z = np.linspace(-30, 30, 601)
    e0 = abs(float(R.silu(np.array([0.0]))[0]))
    e1 = float(np.max(np.abs(R.silu(z) - R.silu(-z) - z)))
    e2 = _rel(R.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy())
    g = np.random.default_rng(5).standard_normal((4, 7))
    e3 = _rel(R.swiglu(g, np.ones_like(g)), R.silu(g))
    e4 = _rel(R.swiglu(g, 2 * np.ones_like(g)),
              2 * torch.nn.functional.silu(torch.from_numpy(g)).numpy())
    return _ok(max(e0, e1, e2, e3, e4), 1e-13, "silu/swiglu closed forms and torch")


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def pin_rope_closed_forms():
    hd, theta = 4, 10000.0
    cos, sin = R.rope_tables(8, hd, theta)
    # pair 0 turns by p radians, pair 1 by p / 100 (theta^(-2/4) = 1/100)
    e = max(abs(cos[3, 0] - math.cos(3.0)), abs(sin[3, 0] - math.sin(3.0)),
            abs(cos[5, 1] - math.cos(0.05)), abs(sin[5, 1] - math.sin(0.05)))
    y = np.array([[1.0, 0.0, 0.0, 0.0]] * 2)  # a = 1, b = 0 in pair 0
    out = R.apply_rope(y, np.array([0, 2]), 1, hd, cos, sin)
    # position 0 is the identity; position 2 turns (1, 0) into (cos 2, sin 2)
    e = max(e, float(np.max(np.abs(out[0] - y[0]))),
            abs(out[1, 0] - math.cos(2.0)), abs(out[1, 2] - math.sin(2.0)))
    return _ok(e, 1e-15, "rope closed forms")


def pin_rope_torch_complex(seed=6):
    """RoPE as complex multiplication: (a + ib) * e^{i angle}, at a small head
    and at the heads of 64 and 128 the kernels take (theta 5e5 and 1e4)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (M, hd, nh, theta) in ((11, 8, 3, 500000.0), (7, 64, 3, 500000.0), (5, 128, 3, 10000.0)):
        y = rng.standard_normal((M, nh * hd))
        pos = rng.integers(0, 2048, size=M)
        cos, sin = R.rope_tables(2048, hd, theta)
        out = R.apply_rope(y, pos, 2, hd, cos, sin)
        yt = torch.from_numpy(y).view(M, nh, 2, hd // 2)
        z = torch.complex(yt[:, :, 0], yt[:, :, 1])
        inv = theta ** (-torch.arange(hd // 2, dtype=torch.float64) * 2 / hd)
        ang = torch.from_numpy(pos).double()[:, None] * inv[None, :]
        rot = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
        ref = torch.stack([rot.real, rot.imag], dim=2).reshape(M, nh * hd).numpy()
        ref[:, 2 * hd:] = y[:, 2 * hd:]  # third head not rotated
        worst = max(worst, _rel(out, ref))
    return _ok(worst, 1e-12, "rope vs torch complex (hd 8, 64, 128)")


def pin_rope_relative(seed=7):
    """<R_m q, R_n k> depends only on m - n; rotations keep pair norms."""
    rng = np.random.default_rng(seed)
    hd = 16
    cos, sin = R.rope_tables(200, hd, 500000.0)
    q = rng.standard_normal((1, hd))
    k = rng.standard_normal((1, hd))
    rq = lambda p: R.apply_rope(q, np.array([p]), 1, hd, cos, sin)[0]
    rk = lambda p: R.apply_rope(k, np.array([p]), 1, hd, cos, sin)[0]
    e1 = abs(np.dot(rq(30), rk(10)) - np.dot(rq(150), rk(130)))
    a = rq(77)
    e2 = float(np.max(np.abs(a[:hd // 2] ** 2 + a[hd // 2:] ** 2
                             - (q[0, :hd // 2] ** 2 + q[0, hd // 2:] ** 2))))
    return _ok(max(e1, e2), 1e-12, "rope relative position / norm")


def pin_attn_bruteforce(seed=8):
    rng = random.Random(seed)
    M, K1, d, nq, nkv, hd, eps, theta = 3, 6, 8, 2, 1, 4, 1e-5, 500000.0
    x, res = _rand(rng, M, K1), _rand(rng, M, d)
    w1, wqkv = _rand(rng, d, K1, 0.4), _rand(rng, (nq + 2 * nkv) * hd, d, 0.4)
    gamma = [1.0 + 0.1 * rng.gauss(0, 1) for _ in range(d)]
    pos = [5, 0, 1234]
    y1 = _bf_gemm_nt(x, w1)
    h = [[res[m][n] + y1[m][n] for n in range(d)] for m in range(M)]
    r = [1.0 / math.sqrt(math.fsum(v * v for v in h[m]) / d + eps) for m in range(M)]
    nrm = [[r[m] * h[m][n] * gamma[n] for n in range(d)] for m in range(M)]
    y = _bf_gemm_nt(nrm, wqkv)
    out = [row[:] for row in y]
    for m in range(M):
        for head in range(nq + nkv):
            for i in range(hd // 2):
                ang = pos[m] * theta ** (-2.0 * i / hd)
                a, b = y[m][head * hd + i], y[m][head * hd + i + hd // 2]
                out[m][head * hd + i] = a * math.cos(ang) - b * math.sin(ang)
                out[m][head * hd + i + hd // 2] = b * math.cos(ang) + a * math.sin(ang)
    o = oracle.attn_in_block(np.array(x), np.array(res), np.array(w1), np.array(wqkv),
                             np.array(gamma), eps, np.array(pos), nq, nkv, hd, theta, 2048)
    return _ok(max(_rel(o["qkv"], out), _rel(o["r"], r), _rel(o["h"], h)), 1e-12,
               "attn brute force")


# ---------------------------------------------------------------------------
# attention core and the full layer
# ---------------------------------------------------------------------------

def _qkv_random(rng, M, n_q, n_kv, hd, scale=1.0):
    return rng.standard_normal((M, (n_q + 2 * n_kv) * hd)) * scale


def pin_attention_bruteforce(seed=20):
    """Pure-Python causal grouped-query attention (math.exp, math.fsum) on two
    sequences of 5 rows, 4 q heads over 2 kv heads of 4 features."""
    rng = np.random.default_rng(seed)
    L, n_seq, n_q, n_kv, hd = 5, 2, 4, 2, 4
    M = L * n_seq
    qkv = _qkv_random(rng, M, n_q, n_kv, hd, 1.5)
    o = R.attention_causal_gqa(qkv, L, n_q, n_kv, hd)
    err = 0.0
    for m in range(M):
        s0 = (m // L) * L
        for h in range(n_q):
            g = h // (n_q // n_kv)
            q = qkv[m, h * hd:(h + 1) * hd]
            sc = []
            for j in range(s0, m + 1):
                k = qkv[j, (n_q + g) * hd:(n_q + g + 1) * hd]
                sc.append(math.fsum(float(q[e]) * float(k[e]) for e in range(hd)) / math.sqrt(hd))
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            z = math.fsum(w)
            for e in range(hd):
                vcol = (n_q + n_kv + g) * hd + e
                ref = math.fsum(w[t] * float(qkv[s0 + t, vcol]) for t in range(len(w))) / z
                err = max(err, abs(o[m, h * hd + e] - ref))
    return _ok(err, 1e-12, "attention brute force")


def pin_attention_torch(seed=21):
    """torch's scaled_dot_product_attention (CPU, float64, is_causal, default
    scale 1/sqrt(hd)) with the kv heads repeated for their q-head groups, at a
    small head and at the heads of 64 and 128 the kernels take."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (L, n_seq, n_q, n_kv, hd) in ((17, 3, 6, 2, 8), (9, 2, 4, 1, 64), (7, 2, 2, 2, 128)):
        M = L * n_seq
        qkv = _qkv_random(rng, M, n_q, n_kv, hd)
        o = R.attention_causal_gqa(qkv, L, n_q, n_kv, hd)
        t = torch.from_numpy(qkv).view(n_seq, L, n_q + 2 * n_kv, hd).permute(0, 2, 1, 3)
        q, k, v = t[:, :n_q], t[:, n_q:n_q + n_kv], t[:, n_q + n_kv:]
        rep = n_q // n_kv
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1), is_causal=True)
        ref = ref.permute(0, 2, 1, 3).reshape(M, n_q * hd).numpy()
        worst = max(worst, _rel(o, ref))
    return _ok(worst, 1e-13, "attention vs torch sdpa (hd 8, 64, 128)")


def pin_attention_closed_forms(seed=22):
    """The first query of each sequence sees only its own key, so its output
    is that key's v row; with every key of a kv head equal, the softmax over
    the visible keys is uniform, so query i gets the mean of v over the keys
    0..i of its sequence."""
    rng = np.random.default_rng(seed)
    L, n_seq, n_q, n_kv, hd = 9, 2, 4, 1, 8
    M = L * n_seq
    qkv = _qkv_random(rng, M, n_q, n_kv, hd)
    o = R.attention_causal_gqa(qkv, L, n_q, n_kv, hd)
    vlo = (n_q + n_kv) * hd
    e = 0.0
    for s0 in (0, L):
        for h in range(n_q):
            e = max(e, float(np.max(np.abs(o[s0, h * hd:(h + 1) * hd] - qkv[s0, vlo:vlo + hd]))))
    qkv2 = qkv.copy()
    qkv2[:, n_q * hd:(n_q + 1) * hd] = rng.standard_normal(hd)[None, :]  # one key for all rows
    o2 = R.attention_causal_gqa(qkv2, L, n_q, n_kv, hd)
    for m in range(M):
        s0 = (m // L) * L
        mean = np.mean(qkv2[s0:m + 1, vlo:vlo + hd], axis=0)
        for h in range(n_q):
            e = max(e, float(np.max(np.abs(o2[m, h * hd:(h + 1) * hd] - mean))))
    return _ok(e, 1e-13, "attention closed forms")


def pin_layer_torch(seed=23):
    """The whole layer in torch float64 from library routines: rms_norm,
    rotation as complex multiplication, scaled_dot_product_attention with the
    kv heads repeated, silu."""
    rng = np.random.default_rng(seed)
    L, n_seq, d, K1, ffn, n_q, n_kv, hd = 6, 2, 16, 12, 20, 4, 2, 4
    M, theta, eps = L * n_seq, 500000.0, 1e-5
    a = rng.standard_normal((M, K1))
    res = rng.standard_normal((M, d))
    w_down = rng.standard_normal((d, K1)) / math.sqrt(K1)
    wqkv = rng.standard_normal(((n_q + 2 * n_kv) * hd, d)) / math.sqrt(d)
    wo = rng.standard_normal((d, n_q * hd)) / math.sqrt(n_q * hd)
    wg, wu = (rng.standard_normal((ffn, d)) / math.sqrt(d) for _ in range(2))
    g1, g2 = 1 + 0.1 * rng.standard_normal(d), 1 + 0.1 * rng.standard_normal(d)
    pos = np.arange(M) % L
    o = R.layer_forward(a, res, w_down, wqkv, g1, wo, wg, wu, g2, eps, pos, n_q, n_kv, hd,
                        theta, L)
    T = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))
    h1 = T(res) + T(a) @ T(w_down).T
    n1 = torch.nn.functional.rms_norm(h1, (d,), weight=T(g1), eps=eps)
    y = (n1 @ T(wqkv).T).view(M, n_q + 2 * n_kv, 2, hd // 2)
    inv = theta ** (-torch.arange(hd // 2, dtype=torch.float64) * 2 / hd)
    ang = T(pos)[:, None] * inv[None, :]
    z = torch.complex(y[:, :, 0], y[:, :, 1])
    rot = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    nr = n_q + n_kv
    yr = torch.cat([torch.stack([rot.real, rot.imag], dim=2)[:, :nr], y[:, nr:]], dim=1)
    qkv = yr.reshape(M, (n_q + 2 * n_kv) * hd)
    t = qkv.view(n_seq, L, n_q + 2 * n_kv, hd).permute(0, 2, 1, 3)
    rep = n_q // n_kv
    att = torch.nn.functional.scaled_dot_product_attention(
        t[:, :n_q], t[:, n_q:nr].repeat_interleave(rep, dim=1),
        t[:, nr:].repeat_interleave(rep, dim=1), is_causal=True)
    att = att.permute(0, 2, 1, 3).reshape(M, n_q * hd)
    h2 = h1 + att @ T(wo).T
    n2 = torch.nn.functional.rms_norm(h2, (d,), weight=T(g2), eps=eps)
    out = torch.nn.functional.silu(n2 @ T(wg).T) * (n2 @ T(wu).T)
    err = max(_rel(o["qkv"], qkv.numpy()), _rel(o["o"], att.numpy()), _rel(o["h2"], h2.numpy()),
              _rel(o["out"], out.numpy()))
    return _ok(err, 1e-12, "layer vs torch")


# ---------------------------------------------------------------------------
# LSE / cross entropy
# ---------------------------------------------------------------------------

def pin_ce_bruteforce(seed=9):
    rng = random.Random(seed)
    M, d, V = 4, 5, 13
    x, w = _rand(rng, M, d, 2.0), _rand(rng, V, d)
    labels = [rng.randrange(V) for _ in range(M)]
    z = _bf_gemm_nt(x, w)
    loss = []
    for m in range(M):
        mx = max(z[m])
        lse = mx + math.log(math.fsum(math.exp(v - mx) for v in z[m]))
        loss.append(lse - z[m][labels[m]])
    o = oracle.lm_head_ce(np.array(x), np.array(w), np.array(labels), chunk=3)
    return _ok(_rel(o["loss"], loss), 1e-12, "ce brute force")


def pin_ce_torch(seed=10):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(9, 16, generator=g, dtype=torch.float64) * 2
    w = torch.randn(37, 16, generator=g, dtype=torch.float64)
    lab = torch.randint(0, 37, (9,), generator=g)
    r = torch.rand(9, generator=g, dtype=torch.float64) + 0.5
    ref = torch.nn.functional.cross_entropy(r[:, None] * (x @ w.T), lab, reduction="none")
    ref_lse = torch.logsumexp(r[:, None] * (x @ w.T), dim=1)
    o = oracle.lm_head_ce(x.numpy(), w.numpy(), lab.numpy(), r=r.numpy(), chunk=4)
    return _ok(max(_rel(o["loss"], ref.numpy()), _rel(o["lse"], ref_lse.numpy())), 1e-13,
               "ce vs torch")


def pin_ce_zero_weights():
    """W = 0: every logit is 0, so loss = ln V for every row."""
    V = 128256
    o = oracle.lm_head_ce(np.ones((3, 4)), np.zeros((V, 4)), np.array([0, 5, V - 1]))
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        lnv = float(json.load(f)["ln_128256"])
    return _ok(float(np.max(np.abs(o["loss"] - lnv))), 1e-12, "W = 0 gives ln V")


def pin_ce_ignored_rows(seed=19):
    """Rows whose label lies outside [0, V) carry no loss: torch's
    cross_entropy with ignore_index = -100 (library routine) gives 0 there, and
    the other rows keep their loss; a label of V or more is ignored the same
    way, and every row's lse is the plain log-sum-exp."""
    g = torch.Generator().manual_seed(seed)
    V = 23
    x = torch.randn(8, 6, generator=g, dtype=torch.float64)
    w = torch.randn(V, 6, generator=g, dtype=torch.float64)
    lab = torch.randint(0, V, (8,), generator=g)
    lab[1] = -100
    lab[4] = -100
    ref = torch.nn.functional.cross_entropy(x @ w.T, lab, reduction="none", ignore_index=-100)
    ref_lse = torch.logsumexp(x @ w.T, dim=1).numpy()
    o = oracle.lm_head_ce(x.numpy(), w.numpy(), lab.numpy(), chunk=3)
    err = max(float(np.max(np.abs(o["loss"] - ref.numpy()))), _rel(o["lse"], ref_lse))
    lab2 = lab.numpy().copy()
    lab2[[1, 4]] = [V, V + 7]
    o2 = oracle.lm_head_ce(x.numpy(), w.numpy(), lab2, chunk=5)
    err = max(err, float(np.max(np.abs(o2["loss"] - ref.numpy()))))
    ok = bool(o["loss"][1] == 0.0 and o["loss"][4] == 0.0 and o2["loss"][1] == 0.0
              and np.all(o["loss"][[0, 2, 3, 5, 6, 7]] > 0))
    return _ok(err if ok else 1.0, 1e-13, "ce ignored rows")


def pin_lse_merge(seed=11):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((5, 300)) * 20
    full = torch.logsumexp(torch.from_numpy(z), dim=1).numpy()
    mx, se = R.tile_lse(z, 64)  # 5 tiles, the last one ragged (44 wide)
    T = mx.shape[0]
    e = _rel(R.lse_merge(mx, se), full)
    e = max(e, _rel(R.lse_merge(mx, se, order=list(range(T))[::-1]), full))
    perm = list(rng.permutation(T))
    e = max(e, _rel(R.lse_merge(mx, se, order=perm), full))
    # pairwise tree: merge (0,1), (2,3), then with 4
    def pair(a, b):
        m = np.maximum(a[0], b[0])
        return m, a[1] * np.exp(a[0] - m) + b[1] * np.exp(b[0] - m)
    p01 = pair((mx[0], se[0]), (mx[1], se[1]))
    p23 = pair((mx[2], se[2]), (mx[3], se[3]))
    t = pair(pair(p01, p23), (mx[4], se[4]))
    e = max(e, _rel(t[0] + np.log(t[1]), full))
    # each tile alone: mx_t + ln se_t is that tile's own logsumexp
    for tt in range(T):
        blk = torch.from_numpy(z[:, tt * 64:(tt + 1) * 64])
        e = max(e, _rel(mx[tt] + np.log(se[tt]), torch.logsumexp(blk, dim=1).numpy()))
    # a single tile is plain logsumexp; the identity pair changes nothing
    m1, s1 = R.tile_lse(z, 300)
    e = max(e, _rel(R.lse_merge(m1, s1), full))
    mi = np.vstack([mx, np.full((1, 5), -np.inf)])
    si = np.vstack([se, np.zeros((1, 5))])
    e = max(e, _rel(R.lse_merge(mi, si), full))
    return _ok(e, 1e-13, "lse merge order independence")


def pin_partial_sumsq(seed=12):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((6, 200))
    P = R.partial_sumsq(h, 64)  # 4 tiles, the last 8 wide
    e = _rel(P.sum(axis=0), [math.fsum(v * v for v in row) for row in h])
    e = max(e, _rel(P[3], [math.fsum(v * v for v in row[192:]) for row in h]))
    return _ok(e, 1e-13, "partial sums of squares")


# ---------------------------------------------------------------------------
# fp8 block
# ---------------------------------------------------------------------------

def pin_fp8_block(seed=13):
    """Brute force of the fp8 block on tiny inputs, with e4m3 codes picked at
    random and values decoded from the format definition by hand here."""
    rng = random.Random(seed)
    M, K1, d, ffn, eps = 3, 4, 4, 5, 1e-5

    def dec(c):  # E4M3FN value of a code, written out from the format
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        return s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))

    finite = [c for c in range(256) if (c & 0x7F) != 0x7F and 0x30 <= (c & 0x7F) <= 0x48]
    codes = lambda r, c: [[rng.choice(finite) for _ in range(c)] for _ in range(r)]
    xq, woq, wgq, wuq = codes(M, K1), codes(d, K1), codes(ffn, d), codes(ffn, d)
    sx, swo, swg, swu = 0.5, 0.25, 0.125, 0.375
    res = _rand(rng, M, d)
    val = lambda q, s: [[dec(c) * s for c in row] for row in q]
    y = _bf_gemm_nt(val(xq, sx), val(woq, swo))
    h = [[res[m][n] + y[m][n] for n in range(d)] for m in range(M)]
    r = [1.0 / math.sqrt(math.fsum(v * v for v in h[m]) / d + eps) for m in range(M)]
    amax = max(abs(v) for row in h for v in row)
    s_h = amax / 448.0
    # nearest E4M3 value (ties to even code) by search over all finite codes
    grid = sorted({(dec(c), c) for c in range(256) if (c & 0x7F) != 0x7F})

    def q8(v):
        best = min(grid, key=lambda t: (abs(t[0] - v), t[1] & 1))
        return best[0]
    hh = [[q8(v / s_h) * s_h for v in row] for row in h]
    g = _bf_gemm_nt(hh, val(wgq, swg))
    u = _bf_gemm_nt(hh, val(wuq, swu))
    out = [[_bf_silu(r[m] * g[m][j]) * r[m] * u[m][j] for j in range(ffn)] for m in range(M)]
    o = oracle.fp8_mlp_block(np.array(xq, dtype=np.uint8), sx, np.array(res),
                             np.array(woq, dtype=np.uint8), swo, np.array(wgq, dtype=np.uint8),
                             swg, np.array(wuq, dtype=np.uint8), swu, eps)
    # the chunked full-tensor amax reads the residual as bf16 bit patterns, so
    # the brute force rounds its residual to bf16 for this check
    res_bits = oracle.codecs.bf16_encode(np.array(res))
    res_b = oracle.codecs.bf16_decode(res_bits)
    hb = [[res_b[m][n] + y[m][n] for n in range(d)] for m in range(M)]
    am_ref = max(abs(v) for row in hb for v in row)
    am = oracle.fp8_h_amax(np.array(xq, dtype=np.uint8), sx, res_bits,
                           np.array(woq, dtype=np.uint8), swo, chunk=2)
    return _ok(max(_rel(o["out"], out), _rel(o["h"], h), _rel(o["r"], r),
                   abs(am - am_ref) / am_ref), 1e-12, "fp8 block brute force")


# ---------------------------------------------------------------------------
# backward of the MLP sub-layer
# ---------------------------------------------------------------------------

def _bf_layer_loss(x, res, wo, wg, wu, gamma, eps, wd, dy):
    """sum(next * dy) of the sub-layer next = h + swiglu(...) wd^T, in pure
    Python (the function whose derivative the backward oracle claims to be)."""
    M, d, ffn = len(x), len(wo), len(wg)
    y = _bf_gemm_nt(x, wo)
    h = [[res[m][n] + y[m][n] for n in range(d)] for m in range(M)]
    tot = []
    for m in range(M):
        r = 1.0 / math.sqrt(math.fsum(v * v for v in h[m]) / d + eps)
        nrm = [r * h[m][n] * gamma[n] for n in range(d)]
        g = [math.fsum(nrm[k] * wg[j][k] for k in range(d)) for j in range(ffn)]
        u = [math.fsum(nrm[k] * wu[j][k] for k in range(d)) for j in range(ffn)]
        out = [_bf_silu(g[j]) * u[j] for j in range(ffn)]
        for n in range(d):
            nxt = h[m][n] + math.fsum(out[j] * wd[n][j] for j in range(ffn))
            tot.append(nxt * dy[m][n])
    return math.fsum(tot)


def _layer_inputs(seed, M=3, K1=5, d=4, ffn=6):
    rng = random.Random(seed)
    return dict(x=_rand(rng, M, K1), res=_rand(rng, M, d), wo=_rand(rng, d, K1, 0.5),
                wg=_rand(rng, ffn, d, 0.5), wu=_rand(rng, ffn, d, 0.5),
                gamma=[1.0 + 0.1 * rng.gauss(0, 1) for _ in range(d)], eps=1e-3,
                wd=_rand(rng, d, ffn, 0.5), dy=_rand(rng, M, d))


def _oracle_bwd(p):
    a = lambda k: np.array(p[k], dtype=np.float64)
    return oracle.mlp_layer_bwd(a("x"), a("res"), a("wo"), a("wg"), a("wu"), a("gamma"),
                                p["eps"], a("wd"), a("dy"))


def pin_swiglu_grad(seed=14):
    """Central differences of silu(g) u, torch float64 autograd, and the
    closed form at g = 0 (silu'(0) = 1/2, silu(0) = 0)."""
    rng = np.random.default_rng(seed)
    g, u, dout = (rng.standard_normal((3, 5)) * 3 for _ in range(3))
    dg, du = R.swiglu_grad(dout, g, u)
    step = 1e-6
    fd_g = np.array([[(_bf_silu(g[i, j] + step) - _bf_silu(g[i, j] - step)) / (2 * step)
                      * u[i, j] * dout[i, j] for j in range(5)] for i in range(3)])
    fd_u = np.array([[_bf_silu(g[i, j]) * dout[i, j] for j in range(5)] for i in range(3)])
    e1 = max(_rel(dg, fd_g), _rel(du, fd_u))
    tg = torch.from_numpy(g).requires_grad_(True)
    tu = torch.from_numpy(u).requires_grad_(True)
    (torch.nn.functional.silu(tg) * tu * torch.from_numpy(dout)).sum().backward()
    e2 = max(_rel(dg, tg.grad.numpy()), _rel(du, tu.grad.numpy()))
    z = np.zeros((1, 4))
    dg0, du0 = R.swiglu_grad(np.full((1, 4), 3.0), z, np.arange(4.0)[None, :])
    e3 = float(np.max(np.abs(dg0 - 1.5 * np.arange(4.0)))) + float(np.max(np.abs(du0)))
    return _ok(max(e1 / 1e3, e2, e3), 1e-12, "swiglu grad (fd/1e3, torch, g=0)")


def pin_layer_bwd_finite_differences(seed=15):
    """Every entry of dx and dres against central differences of the
    pure-Python sub-layer loss sum(next * dy) (step 1e-6: error ~1e-9)."""
    p = _layer_inputs(seed)
    o = _oracle_bwd(p)
    step = 1e-6
    errs = []
    for key, grad in (("x", o["dx"]), ("res", o["dres"]), ("wo", o["dwo"]), ("wg", o["dwg"]),
                      ("wu", o["dwu"]), ("wd", o["dwd"])):
        fd = np.zeros_like(grad)
        for i in range(grad.shape[0]):
            for j in range(grad.shape[1]):
                hi = {**p, key: [row[:] for row in p[key]]}
                lo = {**p, key: [row[:] for row in p[key]]}
                hi[key][i][j] += step
                lo[key][i][j] -= step
                fd[i, j] = (_bf_layer_loss(**hi) - _bf_layer_loss(**lo)) / (2 * step)
        errs.append(_rel(grad, fd))
    fd = np.zeros(len(p["gamma"]))
    for j in range(len(fd)):
        hi, lo = dict(p), dict(p)
        hi["gamma"] = [v + (step if k == j else 0.0) for k, v in enumerate(p["gamma"])]
        lo["gamma"] = [v - (step if k == j else 0.0) for k, v in enumerate(p["gamma"])]
        fd[j] = (_bf_layer_loss(**hi) - _bf_layer_loss(**lo)) / (2 * step)
    errs.append(_rel(o["dgamma"], fd))
    return _ok(max(errs), 1e-7, "layer backward (activations and weights) vs finite differences")


def pin_layer_bwd_torch(seed=16):
    """dout, dg, du, dn, dh and dx against torch float64 autograd of the same
    sub-layer built from library routines (torch rms_norm and silu)."""
    rng = np.random.default_rng(seed)
    M, K1, d, ffn, eps = 5, 12, 8, 10, 1e-5
    t = lambda *s, sc=1.0: torch.from_numpy(rng.standard_normal(s) * sc).requires_grad_(True)
    x, res = t(M, K1), t(M, d)
    wo, wg, wu, wd = t(d, K1, sc=0.3), t(ffn, d, sc=0.3), t(ffn, d, sc=0.3), t(d, ffn, sc=0.3)
    gamma = torch.from_numpy(1 + 0.1 * rng.standard_normal(d))
    dy = torch.from_numpy(rng.standard_normal((M, d)))
    gamma.requires_grad_(True)
    h = res + x @ wo.T
    xh = torch.nn.functional.rms_norm(h, (d,), eps=eps)
    n = xh * gamma
    g, u = n @ wg.T, n @ wu.T
    out = torch.nn.functional.silu(g) * u
    for v in (n, g, u, out, h):
        v.retain_grad()
    gamma.requires_grad_(True)
    ((h + out @ wd.T) * dy).sum().backward()
    num = lambda v: v.detach().numpy()
    o = oracle.mlp_layer_bwd(num(x), num(res), num(wo), num(wg), num(wu), num(gamma), eps,
                             num(wd), dy.numpy())
    errs = [_rel(o["dout"], out.grad.numpy()), _rel(o["dg"], g.grad.numpy()),
            _rel(o["du"], u.grad.numpy()), _rel(o["dn"], n.grad.numpy()),
            _rel(o["dh"], res.grad.numpy()), _rel(o["dx"], x.grad.numpy()),
            _rel(o["dwd"], wd.grad.numpy()), _rel(o["dwg"], wg.grad.numpy()),
            _rel(o["dwu"], wu.grad.numpy()), _rel(o["dwo"], wo.grad.numpy()),
            _rel(o["dgamma"], gamma.grad.numpy())]
    return _ok(max(errs), 1e-12, "layer backward (activations and weights) vs torch autograd")


def pin_rmsnorm_bwd_scale_invariance(seed=17):
    """With eps = 0, RMSNorm is invariant to scaling h, so its gradient is
    orthogonal to h: sum_j dh_j h_j = 0 on every row."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((6, 20)) * rng.uniform(0.2, 5, size=(6, 1))
    dn = rng.standard_normal((6, 20))
    gamma = 1 + 0.1 * rng.standard_normal(20)
    dh, _ = R.rmsnorm_bwd(dn, h, gamma, 0.0)
    dots = np.abs(np.sum(dh * h, axis=1)) / (np.linalg.norm(dh, axis=1) * np.linalg.norm(h, axis=1))
    return _ok(float(np.max(dots)), 1e-13, "rmsnorm backward orthogonal to h")


def pin_bwd_row_coefficient(seed=18):
    """The row coefficient of the RMSNorm backward equals r^2/d times the
    row sum of dz * z over the gate and up pre-activations (z = r h W'^T with
    gamma folded into W', so sum_j h_j G_j = sum_n dz_n z_n / r), the form in
    which a SwiGLU-backward GEMM epilogue can emit it as a partial sum."""
    p = _layer_inputs(seed, M=4, K1=6, d=5, ffn=7)
    o = _oracle_bwd(p)
    d = len(p["wo"])
    alt = o["r"] ** 2 / d * np.sum(o["dg"] * o["g"] + o["du"] * o["u"], axis=1)
    return _ok(_rel(o["coef"], alt), 1e-12, "row coefficient from dz . z")


ALL_PINS = [
    pin_mlp_bruteforce, pin_mlp_exact_example, pin_rmsnorm_torch, pin_rms_closed_forms,
    pin_unit_rms, pin_rowscale_commutes, pin_swiglu, pin_rope_closed_forms,
    pin_rope_torch_complex, pin_rope_relative, pin_attn_bruteforce, pin_attention_bruteforce,
    pin_attention_torch, pin_attention_closed_forms, pin_layer_torch, pin_ce_bruteforce,
    pin_ce_torch, pin_ce_zero_weights, pin_ce_ignored_rows, pin_lse_merge, pin_partial_sumsq, pin_fp8_block,
    pin_swiglu_grad, pin_layer_bwd_finite_differences, pin_layer_bwd_torch,
    pin_rmsnorm_bwd_scale_invariance, pin_bwd_row_coefficient,
]


def run_all():
    """Run every pin; returns list of (name, ok, detail)."""
    out = []
    for p in ALL_PINS:
        try:
            ok, detail = p()
        except Exception as e:  # a broken oracle may raise instead of erring
            ok, detail = False, f"raised {type(e).__name__}: {e}"
        out.append((p.__name__, ok, detail))
    return out

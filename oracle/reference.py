"""Plain fp64 definitions of the hot path (TEST INFRASTRUCTURE ONLY).

Citations name sections of the news page "CODA: New Research Optimizes
Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).

Everything is unfused and in float64 on the exact input values.  Weights are
stored [N, K] (row n holds output feature n), so a linear layer is x @ W^T.
Every block is row-independent: callers may pass a subset of token rows and get
exactly the corresponding rows of the full result.  That is how full-size
configurations are checked on sampled rows.
"""

import numpy as np


# ---------------------------------------------------------------------------
# building blocks
# ---------------------------------------------------------------------------

def gemm_nt(a, w):
    """y = a @ w^T for a [M,K], w [N,K] (the blocked multiply the page calls
    the GEMM mainloop, section "CODA: the secret in the epilogue").  float64
    BLAS is used as the library matmul step."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return a @ w.T


def residual_add(y, res):
    """h = res + y (elementwise residual add; section "Five building blocks
    and a LEGO language", elementwise transform)."""
    return np.asarray(res, dtype=np.float64) + np.asarray(y, dtype=np.float64)


def rms_scale(h, eps):
    """Per-row RMS scale r[m] = 1 / sqrt(mean_n h[m,n]^2 + eps).

    The page (section "CODA: the secret in the epilogue") calls this the row
    scale factor of RMS normalisation; it prints no formula.  Reading: eps
    inside the square root, mean over the row's N features."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=1)
    return 1.0 / np.sqrt(ms + eps)


def rmsnorm(h, gamma, eps):
    """RMSNorm applied before the second GEMM (the unfused form):
    n = diag(r) . h . diag(gamma)."""
    r = rms_scale(h, eps)
    return (r[:, None] * np.asarray(h, dtype=np.float64)) * np.asarray(gamma, dtype=np.float64)[None, :]


def silu(z):
    """silu(z) = z / (1 + exp(-z)) (the SiLU gate of SwiGLU)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    """SwiGLU activation: silu(g) * u with g the gate projection and u the up
    projection (named in sections "The cost of laziness..." and "CODA: the
    secret in the epilogue"; reading: the LLaMA form)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


# ---------------------------------------------------------------------------
# MLP block: GEMM -> residual -> RMSNorm -> GEMM (gate|up) -> SwiGLU
# ---------------------------------------------------------------------------

def mlp_block(x, res, wo, wg, wu, gamma, eps):
    """GEMM-RMSNorm-GEMM with SwiGLU, unfused (section "CODA: the secret in
    the epilogue": a matmul, a residual add, RMS normalisation, then a second
    matmul; the SwiGLU step applies the same scheme).

    x [M,K1], res [M,d], wo [d,K1], wg/wu [ffn,d], gamma [d] -> dict with
      h   [M,d]   = res + x wo^T
      r   [M]     = rms_scale(h)
      g,u [M,ffn] = (diag(r) h diag(gamma)) wg^T, ... wu^T
      out [M,ffn] = silu(g) * u
    """
    h = residual_add(gemm_nt(x, wo), res)
    r = rms_scale(h, eps)
    n = (r[:, None] * h) * np.asarray(gamma, dtype=np.float64)[None, :]
    g = gemm_nt(n, wg)
    u = gemm_nt(n, wu)
    return {"h": h, "r": r, "g": g, "u": u, "out": swiglu(g, u)}


# ---------------------------------------------------------------------------
# Backward of the MLP sub-layer.  Section "CODA: the secret in the epilogue"
# states that when the tail of the forward pass is block-local the backward
# pass inherits the same structure, and section "Experimental results" reports backward
# kernels for GEMM-Residual-PartialRMS-GEMM and for SwiGLU.  The page prints
# no formulas: what follows is the chain rule applied to the forward
# definitions above, in the order the forward computes.
# ---------------------------------------------------------------------------

def swiglu_grad(dout, g, u):
    """Gradients of out = silu(g) * u given dout = dL/dout:
    du = dout * silu(g) and dg = dout * u * silu'(g), where, with
    s = 1 / (1 + exp(-g)), silu'(g) = s + g s (1 - s)."""
    dout = np.asarray(dout, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    dsilu = s + g * s * (1.0 - s)
    return dout * u * dsilu, dout * (g * s)


def rmsnorm_bwd(dn, h, gamma, eps):
    """Gradient w.r.t. h of n = r h gamma, r = (mean_j h_j^2 + eps)^(-1/2),
    given dn = dL/dn.  Per row, d r / d h_j = -r^3 h_j / d, so
        dh_j = r gamma_j dn_j - (r^3 / d) h_j sum_k gamma_k dn_k h_k.
    Returns (dh, coefficient r^3/d sum_k gamma_k dn_k h_k per row)."""
    h = np.asarray(h, dtype=np.float64)
    dng = np.asarray(dn, dtype=np.float64) * np.asarray(gamma, dtype=np.float64)[None, :]
    r = rms_scale(h, eps)
    d = h.shape[1]
    coef = r ** 3 / d * np.sum(dng * h, axis=1)
    return r[:, None] * dng - coef[:, None] * h, coef


def mlp_layer_bwd(x, res, wo, wg, wu, gamma, eps, wd, dy):
    """Backward of the MLP sub-layer of a pre-norm block,
        h = res + x wo^T,  out = mlp_block(...)["out"],  next = h + out wd^T,
    given dy = dL/dnext [M,d] (wd [d,ffn] is the down projection).

    Returns the forward values of mlp_block plus
      dout [M,ffn] = dy wd                    (through the down projection)
      dg, du       = swiglu_grad(dout, g, u)
      dn   [M,d]   = dg wg + du wu            (gradient w.r.t. n = r h gamma)
      dh   [M,d]   = rmsnorm_bwd(dn, h) + dy  (the skip connection adds dy)
      coef [M]     = the per-row coefficient of rmsnorm_bwd
      dres = dh,  dx [M,K1] = dh wo           (h = res + x wo^T)
    and the weight gradients (sums over the token rows):
      dwd [d,ffn]  = dy^T out                 (next = h + out wd^T)
      dwg, dwu [ffn,d] = dg^T n, du^T n       (g = n wg^T, n = r h gamma)
      dgamma [d]   = sum_m dn (r h)           (n_j = (r h)_j gamma_j)
      dwo [d,K1]   = dh^T x
    """
    f = mlp_block(x, res, wo, wg, wu, gamma, eps)
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    dout = dy @ np.asarray(wd, dtype=np.float64)
    dg, du = swiglu_grad(dout, f["g"], f["u"])
    dn = dg @ np.asarray(wg, dtype=np.float64) + du @ np.asarray(wu, dtype=np.float64)
    dh_norm, coef = rmsnorm_bwd(dn, f["h"], gamma, eps)
    dh = dh_norm + dy
    dx = dh @ np.asarray(wo, dtype=np.float64)
    rh = f["r"][:, None] * f["h"]
    n = rh * np.asarray(gamma, dtype=np.float64)[None, :]
    f.update({"dout": dout, "dg": dg, "du": du, "dn": dn, "coef": coef, "dh": dh,
              "dres": dh, "dx": dx,
              "dwd": dy.T @ f["out"], "dwg": dg.T @ n, "dwu": du.T @ n,
              "dgamma": np.sum(dn * rh, axis=0), "dwo": dh.T @ x})
    return f


def fp8_mlp_block(xq, sx, res, woq, swo, wgq, swg, wuq, swu, eps, h_scale=None):
    """The same block with e4m3 operands (section "The cost of laziness in
    large-model training" names FP8 as the regime where data movement
    dominates).

    xq [M,K1], woq [d,K1], wgq/wuq [ffn,d] are E4M3FN codes (uint8), each with
    one fp32 per-tensor scale (value = decode(code) * scale); res [M,d] is the
    residual's float64 value.  gamma was folded into wg/wu before they were
    quantised, so it does not appear here.

    The second GEMM reads h as e4m3 too.  That rounding is part of what an fp8
    GEMM computes, so the oracle models it once:
      s_h   = max|h| / 448 from the unrounded h (current scaling), unless a
              scale is given,
      h_hat = s_h * E4M3(h / s_h)   (round to nearest even, saturating)
      g, u  = r * (h_hat Wg^T), r * (h_hat Wu^T);  out = silu(g) * u.
    """
    from .codecs import e4m3_decode, e4m3_encode_fast, E4M3_MAX

    x = e4m3_decode(xq) * float(sx)
    wo = e4m3_decode(woq) * float(swo)
    h = residual_add(gemm_nt(x, wo), res)
    r = rms_scale(h, eps)
    amax = float(np.max(np.abs(h)))
    s_h = amax / E4M3_MAX if h_scale is None else float(h_scale)
    h_hat = e4m3_decode(e4m3_encode_fast(h / s_h)) * s_h
    g = r[:, None] * gemm_nt(h_hat, e4m3_decode(wgq) * float(swg))
    u = r[:, None] * gemm_nt(h_hat, e4m3_decode(wuq) * float(swu))
    return {"h": h, "r": r, "amax": amax, "s_h": s_h, "h_hat": h_hat,
            "g": g, "u": u, "out": swiglu(g, u)}


def fp8_h_amax(xq, sx, res_bits, woq, swo, chunk=1024):
    """max |h| over every row of h = res + x W1^T for the fp8 block, in row
    chunks (the per-tensor scale of h is chosen from it: s_h = amax / 448).
    res_bits are the residual's bf16 bit patterns."""
    from .codecs import e4m3_decode, bf16_decode

    wo = e4m3_decode(woq) * float(swo)
    amax = 0.0
    for m0 in range(0, xq.shape[0], chunk):
        x = e4m3_decode(xq[m0:m0 + chunk]) * float(sx)
        h = residual_add(gemm_nt(x, wo), bf16_decode(res_bits[m0:m0 + chunk]))
        amax = max(amax, float(np.max(np.abs(h))))
    return amax


# ---------------------------------------------------------------------------
# attention-input block: GEMM -> residual -> RMSNorm -> QKV GEMM -> RoPE
# ---------------------------------------------------------------------------

def rope_tables(max_pos, head_dim, theta):
    """cos/sin of the rotary angles, [max_pos, head_dim/2] float64.

    Rotary position embedding is named (section "CODA: the secret in the
    epilogue") without a formula.  Reading: angle(p, i) = p * theta^(-2i/hd)
    for i = 0 .. hd/2-1, no frequency rescaling."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(y, pos, n_rot_heads, head_dim, cos, sin):
    """Rotate the first n_rot_heads heads of y [M, heads*hd] by position.

    Rotate-half pairing: within a head, feature i pairs with i + hd/2:
      (a, b) -> (a cos - b sin, b cos + a sin).
    Heads past n_rot_heads (the v heads) are returned unchanged."""
    y = np.array(y, dtype=np.float64, copy=True)
    half = head_dim // 2
    c = cos[np.asarray(pos)]  # [M, half]
    s = sin[np.asarray(pos)]
    for hh in range(n_rot_heads):
        lo = hh * head_dim
        a = y[:, lo:lo + half].copy()
        b = y[:, lo + half:lo + head_dim].copy()
        y[:, lo:lo + half] = a * c - b * s
        y[:, lo + half:lo + head_dim] = b * c + a * s
    return y


def attn_in_block(a, res, w1, wqkv, gamma, eps, pos, n_q, n_kv, head_dim, theta,
                  max_pos):
    """GEMM-RMSNorm-GEMM feeding attention, with RoPE on q and k.

    a [M,K1], res [M,d], w1 [d,K1], wqkv [(n_q+2 n_kv) hd, d], gamma [d],
    pos [M] -> dict(h, r, qkv [M, (n_q+2 n_kv) hd] laid out q | k | v)."""
    h = residual_add(gemm_nt(a, w1), res)
    r = rms_scale(h, eps)
    n = (r[:, None] * h) * np.asarray(gamma, dtype=np.float64)[None, :]
    y = gemm_nt(n, wqkv)
    cos, sin = rope_tables(max_pos, head_dim, theta)
    qkv = apply_rope(y, pos, n_q + n_kv, head_dim, cos, sin)
    return {"h": h, "r": r, "qkv": qkv}


# ---------------------------------------------------------------------------
# attention core and the full layer (section "What CODA can do": every
# operator of the layer except attention and the embedding is re-parameterised;
# attention itself is the plain definition here, needed for the layer forward)
# ---------------------------------------------------------------------------

def attention_causal_gqa(qkv, seq_len, n_q, n_kv, head_dim):
    """Causal grouped-query softmax attention.

    qkv [M, (n_q + 2 n_kv) hd] laid out q | k | v, hd features per head; rows
    [s L, (s+1) L) form sequence s (L = seq_len).  Reading (the page gives no
    attention formula; this is the standard causal form): q head h attends
    with kv head h // (n_q / n_kv); the score of query i and key j is
    q_i . k_j / sqrt(hd); key j is visible to query i iff both lie in the same
    sequence and j <= i; o_i = sum_j softmax_j(score_ij) v_j.
    Returns o [M, n_q hd]."""
    qkv = np.asarray(qkv, dtype=np.float64)
    M = qkv.shape[0]
    hd = head_dim
    group = n_q // n_kv
    o = np.empty((M, n_q * hd))
    visible = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for s0 in range(0, M, seq_len):
        rows = slice(s0, s0 + seq_len)
        for h in range(n_q):
            g = h // group
            q = qkv[rows, h * hd:(h + 1) * hd]
            k = qkv[rows, (n_q + g) * hd:(n_q + g + 1) * hd]
            v = qkv[rows, (n_q + n_kv + g) * hd:(n_q + n_kv + g + 1) * hd]
            sc = np.where(visible, (q @ k.T) / np.sqrt(hd), -np.inf)
            p = np.exp(sc - np.max(sc, axis=1, keepdims=True))
            o[rows, h * hd:(h + 1) * hd] = (p / np.sum(p, axis=1, keepdims=True)) @ v
    return o


def layer_forward(a, res, w_down, wqkv, gamma1, wo, wg, wu, gamma2, eps, pos, n_q, n_kv,
                  head_dim, theta, seq_len):
    """One pre-norm transformer layer, in the periodic form of the hot path
    (each GEMM output that feeds an RMSNorm is a residual add):
      h1  = res + a w_down^T             (the previous MLP's down projection)
      qkv = RoPE(RMSNorm(h1; gamma1) wqkv^T) on the q and k heads
      o   = attention_causal_gqa(qkv)
      h2  = h1 + o wo^T                  (attention output projection)
      out = SwiGLU(RMSNorm(h2; gamma2) wg^T, RMSNorm(h2; gamma2) wu^T)
    out is what the layer's own down projection reads next.
    Returns dict(h1, r1, qkv, o, h2, r2, out)."""
    f1 = attn_in_block(a, res, w_down, wqkv, gamma1, eps, pos, n_q, n_kv, head_dim, theta,
                       seq_len)
    o = attention_causal_gqa(f1["qkv"], seq_len, n_q, n_kv, head_dim)
    f2 = mlp_block(o, f1["h"], wo, wg, wu, gamma2, eps)
    return {"h1": f1["h"], "r1": f1["r"], "qkv": f1["qkv"], "o": o, "h2": f2["h"],
            "r2": f2["r"], "out": f2["out"]}


# ---------------------------------------------------------------------------
# LM head cross entropy via log-sum-exp
# ---------------------------------------------------------------------------

def logsumexp_rows(z):
    """lse[m] = max_n z + ln sum_n exp(z - max) (natural log)."""
    z = np.asarray(z, dtype=np.float64)
    mx = np.max(z, axis=1)
    return mx + np.log(np.sum(np.exp(z - mx[:, None]), axis=1))


def lm_head_ce(x, wlm, labels, r=None, chunk=256):
    """Per-row cross entropy of the LM head (section "CODA: the secret in the
    epilogue" lists cross-entropy among the re-parameterised ops).

    z = diag(r) x wlm^T (r optional), loss[m] = lse(z[m]) - z[m, label[m]].
    Reading (the page is silent on it): a label outside [0, V), such as an
    ignore index of -100, marks a row that carries no loss, so loss[m] = 0;
    its lse is still defined and its label logit is NaN.
    Rows are processed in chunks so the float64 logits stay bounded."""
    x = np.asarray(x, dtype=np.float64)
    labels = np.asarray(labels)
    M = x.shape[0]
    V = np.asarray(wlm).shape[0]
    valid = (labels >= 0) & (labels < V)
    lse = np.empty(M)
    zl = np.full(M, np.nan)
    for m0 in range(0, M, chunk):
        z = gemm_nt(x[m0:m0 + chunk], wlm)
        if r is not None:
            z = np.asarray(r, dtype=np.float64)[m0:m0 + chunk, None] * z
        lse[m0:m0 + chunk] = logsumexp_rows(z)
        rows = np.nonzero(valid[m0:m0 + chunk])[0]
        zl[m0 + rows] = z[rows, labels[m0 + rows]]
    loss = np.where(valid, lse - np.where(valid, zl, 0.0), 0.0)
    return {"lse": lse, "label_logit": zl, "loss": loss}


# ---------------------------------------------------------------------------
# block-local quantities the epilogues emit (section "Five building blocks and
# a LEGO language": block reduction -- local RMS, block log-sum-exp; stateful
# transform -- running max and sum-exp)
# ---------------------------------------------------------------------------

def partial_sumsq(h, width):
    """P[t, m] = sum over columns [t*width, (t+1)*width) of h[m, n]^2."""
    h = np.asarray(h, dtype=np.float64)
    M, N = h.shape
    T = (N + width - 1) // width
    P = np.zeros((T, M))
    for t in range(T):
        blk = h[:, t * width:(t + 1) * width]
        P[t] = np.sum(blk * blk, axis=1)
    return P


def tile_lse(z, width):
    """Per (tile, row) (max, sum exp(z - max)) over columns of width `width`.
    Returns mx [T, M], se [T, M]."""
    z = np.asarray(z, dtype=np.float64)
    M, V = z.shape
    T = (V + width - 1) // width
    mx = np.empty((T, M))
    se = np.empty((T, M))
    for t in range(T):
        blk = z[:, t * width:(t + 1) * width]
        mx[t] = np.max(blk, axis=1)
        se[t] = np.sum(np.exp(blk - mx[t][:, None]), axis=1)
    return mx, se


def lse_merge(mx, se, order=None):
    """Combine per-tile (max, sum-exp) pairs into lse, one pair at a time in
    the given tile order (the online-normalisation statistics).  The pair
    (-inf, 0) is the identity of the merge."""
    mx = np.asarray(mx, dtype=np.float64)
    se = np.asarray(se, dtype=np.float64)
    T = mx.shape[0]
    order = range(T) if order is None else order
    run_m = np.full(mx.shape[1], -np.inf)
    run_s = np.zeros(mx.shape[1])
    for t in order:
        new_m = np.maximum(run_m, mx[t])
        with np.errstate(invalid="ignore"):
            a = np.where(run_s > 0, run_s * np.exp(run_m - new_m), 0.0)
            b = np.where(se[t] > 0, se[t] * np.exp(mx[t] - new_m), 0.0)
        run_m, run_s = new_m, a + b
    return run_m + np.log(run_s)

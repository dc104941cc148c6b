"""Seeded synthetic inputs for the hot path's workloads.

This module holds no arithmetic of the method itself: it only draws random
numbers and rounds them to the storage formats the kernels read (bf16, OCP
E4M3FN with one fp32 scale per tensor).  Both the HIP path and the CPU oracle
receive the arrays built here; neither builds its own.

Every tensor has its own streams, one per chunk of about 2^20 elements (whole
rows):
    numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=(workload, tensor, chunk))))
so tensors are reproducible independently of each other, of generation order
and of the number of threads that draw the chunks.  Normals are drawn in float32 and scaled by their standard deviation,
then rounded to bf16 (round to nearest even, via torch's CPU cast) or
quantised to e4m3 with scale = amax / 448 (torch's CPU cast after clamping, so
that the code saturates instead of overflowing to NaN).

The shapes and distributions follow the LLaMA-3-shaped workloads:
  mlp_tiny   M=64,    d=256,  K1=256,  ffn=512   (bf16)
  mlp_1b     M=8192,  d=2048, K1=2048, ffn=8192  (bf16)
  attn_rope  M=8192,  d=2048, K1=8192, 32 q / 8 kv heads of 64, theta 5e5
  lm_head    M=8192,  d=2048, V=128256
  mlp_8b_fp8 M=16384, d=4096, K1=4096, ffn=14336 (e4m3)
  mlp_7b     M=8192,  d=4096, K1=4096, ffn=11008 (bf16)
  mlp_70b    M=8192,  d=8192, K1=8192, ffn=28672 (bf16)
  mlp_1b_bwd as mlp_1b, plus down projection wd and output gradient dy
  layer_1b   one transformer layer at the 1B shape: the attn_rope block (the
             previous MLP's down projection, K1=8192, then QKV + RoPE), causal
             grouped-query attention over 4 sequences of 2048, then the mlp_1b
             block with the attention output projection wo as its GEMM1
  layer_7b   the layer at d=4096, K1=ffn=11008, 32 q / 32 kv heads of 128
  layer_70b  the layer at d=8192, K1=ffn=28672, 64 q / 8 kv heads of 128
Activations and residuals ~ N(0, 1); weights ~ N(0, 1/fan_in of the layer
they feed, i.e. 1/d for the d-wide layers); gamma = 1 + 0.1 N(0, 1).
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0

WORKLOADS = {
    # name: (workload id, kind, sizes)
    "mlp_tiny": (0, "mlp", dict(M=64, d=256, K1=256, ffn=512)),
    "mlp_1b": (1, "mlp", dict(M=8192, d=2048, K1=2048, ffn=8192)),
    "attn_rope": (2, "attn", dict(M=8192, d=2048, K1=8192, n_q=32, n_kv=8, head_dim=64,
                                  theta=500000.0, seq_len=2048)),
    "lm_head": (3, "lm", dict(M=8192, d=2048, V=128256)),
    "mlp_8b_fp8": (4, "mlp_fp8", dict(M=16384, d=4096, K1=4096, ffn=14336)),
    # the same MLP block at the 7B and 70B hidden sizes (LLaMA-2-7B: d=4096,
    # ffn=11008; LLaMA-2/3-70B: d=8192, ffn=28672), M=8192 tokens as for 1B
    "mlp_7b": (5, "mlp", dict(M=8192, d=4096, K1=4096, ffn=11008)),
    "mlp_70b": (6, "mlp", dict(M=8192, d=8192, K1=8192, ffn=28672)),
    # forward + backward of the 1B-shaped MLP sub-layer (adds the down
    # projection and the gradient arriving at the sub-layer's output)
    "mlp_1b_bwd": (7, "mlp_bwd", dict(M=8192, d=2048, K1=2048, ffn=8192)),
    # one transformer layer (attention input block -> attention -> MLP block)
    "layer_1b": (8, "layer", dict(M=8192, d=2048, K1=8192, ffn=8192, n_q=32, n_kv=8,
                                  head_dim=64, theta=500000.0, seq_len=2048)),
    # the same layer at the 7B and 70B hidden sizes: LLaMA-2-7B (32 heads of
    # 128, no grouping, RoPE theta 1e4, ffn 11008) and LLaMA-3-70B (64 q / 8 kv
    # heads of 128, theta 5e5, ffn 28672); the previous MLP's width is ffn
    "layer_7b": (9, "layer", dict(M=8192, d=4096, K1=11008, ffn=11008, n_q=32, n_kv=32,
                                  head_dim=128, theta=10000.0, seq_len=2048)),
    "layer_70b": (10, "layer", dict(M=8192, d=8192, K1=28672, ffn=28672, n_q=64, n_kv=8,
                                    head_dim=128, theta=500000.0, seq_len=2048)),
}

_TENSOR_IDS = {"x": 0, "res": 1, "w1": 2, "wg": 3, "wu": 4, "gamma": 5, "wqkv": 6,
               "wlm": 7, "labels": 8, "wd": 9, "dy": 10, "wo": 11, "gamma2": 12}


def _rng(seed, workload_id, tensor, chunk=None):
    key = (workload_id, _TENSOR_IDS[tensor]) + (() if chunk is None else (chunk,))
    ss = np.random.SeedSequence(seed, spawn_key=key)
    return np.random.Generator(np.random.PCG64(ss))


_CHUNK_ELEMS = 1 << 20
_POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def normal_f32(seed, workload_id, tensor, shape, std):
    """float32 N(0, std^2) array.  Rows are drawn in chunks of about 2^20
    elements (R = max(1, 2^20 // row length) rows); chunk c (rows
    [R c, R c + R)) has its own stream (spawn key (workload, tensor, c)), so
    the chunks are drawn in parallel threads and the values do not depend on
    the thread count."""
    out = np.empty(shape, dtype=np.float32)
    rows = shape[0]
    row_elems = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    chunk_rows = max(1, _CHUNK_ELEMS // row_elems)

    def fill(c):
        r0, r1 = c * chunk_rows, min(rows, (c + 1) * chunk_rows)
        blk = out[r0:r1]
        _rng(seed, workload_id, tensor, c).standard_normal(out=blk, dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)

    list(_POOL.map(fill, range((rows + chunk_rows - 1) // chunk_rows)))
    return out


def to_bf16_bits(a32):
    """float32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3(a32):
    """float32 array -> (uint8 E4M3FN codes, fp32 scale) with scale = amax/448."""
    amax = float(np.max(np.abs(a32)))
    scale = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
    t = torch.from_numpy(np.ascontiguousarray(a32)) / float(scale)
    t = torch.clamp(t, -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy(), float(scale)


@dataclass
class Workload:
    """Host copies of one workload's inputs.  bf16 tensors are uint16 bit
    patterns, e4m3 tensors uint8 codes; scales are Python floats."""
    name: str
    kind: str
    sizes: dict
    seed: int
    arrays: dict = field(default_factory=dict)
    scales: dict = field(default_factory=dict)


def make_mlp(seed=0, M=64, d=256, K1=256, ffn=512, workload_id=0, name="mlp"):
    """bf16 MLP block inputs: x [M,K1], res [M,d], w1 [d,K1], wg/wu [ffn,d],
    gamma [d] float32."""
    w = Workload(name, "mlp", dict(M=M, d=d, K1=K1, ffn=ffn), seed)
    w.arrays["x"] = to_bf16_bits(normal_f32(seed, workload_id, "x", (M, K1), 1.0))
    w.arrays["res"] = to_bf16_bits(normal_f32(seed, workload_id, "res", (M, d), 1.0))
    w.arrays["w1"] = to_bf16_bits(normal_f32(seed, workload_id, "w1", (d, K1), d ** -0.5))
    w.arrays["wg"] = to_bf16_bits(normal_f32(seed, workload_id, "wg", (ffn, d), d ** -0.5))
    w.arrays["wu"] = to_bf16_bits(normal_f32(seed, workload_id, "wu", (ffn, d), d ** -0.5))
    g = normal_f32(seed, workload_id, "gamma", (d,), 1.0)
    w.arrays["gamma"] = (np.float32(1.0) + np.float32(0.1) * g).astype(np.float32)
    return w


def make_mlp_bwd(seed=0, M=64, d=256, K1=256, ffn=512, workload_id=7, name="mlp_bwd"):
    """MLP sub-layer inputs for the backward pass: those of make_mlp plus the
    down projection wd [d,ffn] ~ N(0, 1/ffn) and the gradient dy [M,d] ~ N(0,1)
    of the sub-layer output."""
    w = make_mlp(seed, M, d, K1, ffn, workload_id, name)
    w.kind = "mlp_bwd"
    w.arrays["wd"] = to_bf16_bits(normal_f32(seed, workload_id, "wd", (d, ffn), ffn ** -0.5))
    w.arrays["dy"] = to_bf16_bits(normal_f32(seed, workload_id, "dy", (M, d), 1.0))
    return w


def make_attn(seed=0, M=64, d=256, K1=256, n_q=4, n_kv=2, head_dim=64, theta=500000.0,
              seq_len=2048, workload_id=2, name="attn"):
    """Attention-input block inputs: a [M,K1], res [M,d], w1 [d,K1],
    wqkv [(n_q+2 n_kv) hd, d], gamma [d], positions m mod seq_len."""
    nqkv = (n_q + 2 * n_kv) * head_dim
    w = Workload(name, "attn", dict(M=M, d=d, K1=K1, n_q=n_q, n_kv=n_kv, head_dim=head_dim,
                                    theta=theta, seq_len=seq_len), seed)
    w.arrays["x"] = to_bf16_bits(normal_f32(seed, workload_id, "x", (M, K1), 1.0))
    w.arrays["res"] = to_bf16_bits(normal_f32(seed, workload_id, "res", (M, d), 1.0))
    w.arrays["w1"] = to_bf16_bits(normal_f32(seed, workload_id, "w1", (d, K1), d ** -0.5))
    w.arrays["wqkv"] = to_bf16_bits(normal_f32(seed, workload_id, "wqkv", (nqkv, d), d ** -0.5))
    g = normal_f32(seed, workload_id, "gamma", (d,), 1.0)
    w.arrays["gamma"] = (np.float32(1.0) + np.float32(0.1) * g).astype(np.float32)
    w.arrays["pos"] = (np.arange(M, dtype=np.int64) % seq_len).astype(np.int32)
    return w


def make_lm(seed=0, M=64, d=256, V=1000, workload_id=3, name="lm"):
    """LM-head inputs: x [M,d] bf16, wlm [V,d] bf16, labels [M] int32 in [0,V)."""
    w = Workload(name, "lm", dict(M=M, d=d, V=V), seed)
    w.arrays["x"] = to_bf16_bits(normal_f32(seed, workload_id, "x", (M, d), 1.0))
    w.arrays["wlm"] = to_bf16_bits(normal_f32(seed, workload_id, "wlm", (V, d), d ** -0.5))
    w.arrays["labels"] = _rng(seed, workload_id, "labels").integers(0, V, size=M, dtype=np.int32)
    return w


def make_mlp_fp8(seed=0, M=64, d=256, K1=256, ffn=512, workload_id=4, name="mlp_fp8"):
    """fp8 MLP block inputs: e4m3 x [M,K1], w1 [d,K1], wg/wu [ffn,d] with one
    fp32 scale each; bf16 res [M,d].  The weights stand for gate/up weights
    with the RMSNorm gain already folded in, so no gamma is drawn."""
    w = Workload(name, "mlp_fp8", dict(M=M, d=d, K1=K1, ffn=ffn), seed)
    for t, shape, std in (("x", (M, K1), 1.0), ("w1", (d, K1), d ** -0.5),
                          ("wg", (ffn, d), d ** -0.5), ("wu", (ffn, d), d ** -0.5)):
        codes, s = to_e4m3(normal_f32(seed, workload_id, t, shape, std))
        w.arrays[t] = codes
        w.scales[t] = s
    w.arrays["res"] = to_bf16_bits(normal_f32(seed, workload_id, "res", (M, d), 1.0))
    return w


def make_layer(seed=0, M=64, d=256, K1=512, ffn=512, n_q=4, n_kv=2, head_dim=64,
               theta=500000.0, seq_len=32, workload_id=8, name="layer"):
    """One transformer layer in the periodic form of the hot path: the inputs
    of make_attn (x = the previous MLP activation [M,K1], res [M,d], w1 = its
    down projection [d,K1], wqkv, gamma, positions m mod seq_len) plus the
    attention output projection wo [d, n_q hd] ~ N(0, 1/(n_q hd)), the gate and
    up weights wg/wu [ffn,d] ~ N(0, 1/d) and the second RMSNorm gain gamma2."""
    w = make_attn(seed, M, d, K1, n_q, n_kv, head_dim, theta, seq_len, workload_id, name)
    w.kind = "layer"
    w.sizes["ffn"] = ffn
    w.arrays["wo"] = to_bf16_bits(normal_f32(seed, workload_id, "wo", (d, n_q * head_dim),
                                             (n_q * head_dim) ** -0.5))
    w.arrays["wg"] = to_bf16_bits(normal_f32(seed, workload_id, "wg", (ffn, d), d ** -0.5))
    w.arrays["wu"] = to_bf16_bits(normal_f32(seed, workload_id, "wu", (ffn, d), d ** -0.5))
    g = normal_f32(seed, workload_id, "gamma2", (d,), 1.0)
    w.arrays["gamma2"] = (np.float32(1.0) + np.float32(0.1) * g).astype(np.float32)
    return w


def make_workload(name, seed=0, **overrides):
    """Build a named workload at its full sizes (or with sizes overridden)."""
    wid, kind, sizes = WORKLOADS[name]
    sizes = dict(sizes)
    sizes.update(overrides)
    if kind == "mlp":
        return make_mlp(seed, workload_id=wid, name=name, **sizes)
    if kind == "attn":
        return make_attn(seed, workload_id=wid, name=name, **sizes)
    if kind == "lm":
        return make_lm(seed, workload_id=wid, name=name, **sizes)
    if kind == "mlp_bwd":
        return make_mlp_bwd(seed, workload_id=wid, name=name, **sizes)
    if kind == "mlp_fp8":
        return make_mlp_fp8(seed, workload_id=wid, name=name, **sizes)
    if kind == "layer":
        return make_layer(seed, workload_id=wid, name=name, **sizes)
    raise KeyError(name)

"""CPU oracle for the GEMM-epilogue transformer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); the only things both sides
see are the seeded input arrays, which the harness builds and passes in.

Every function here is the plain, unfused definition of what the method
computes, in numpy float64 on the exact values of the (bf16 or e4m3) inputs,
with no blocking, fusion or reordering beyond what the definition states.

Citations name sections of the news page "CODA: New Research Optimizes
Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash; the
same article in Vietnamese, Indonesian and Hindi editions).  The page prints
prose only -- no equations, tables or worked numbers -- so each function says
which reading of that prose it implements.

Pins (what each function is checked against, independently of itself) live in
tests/test_oracle_*.py.  Parity status per function:
  codecs.*                  pinned (exhaustive e4m3 table, bf16 vs torch casts)
  mlp_block / fp8_mlp_block pinned (brute force, exact-rational example,
                            torch rms_norm/silu, commutation identity)
  attn_in_block, rope_*     pinned (brute force, rotation closed forms,
                            relative-position invariant, torch complex mult.)
  attention_causal_gqa      pinned (brute force with math.fsum, torch
                            scaled_dot_product_attention, first-query and
                            equal-key closed forms)
  layer_forward             pinned (torch float64 layer from rms_norm,
                            complex rotation, scaled_dot_product_attention,
                            silu)
  lm_head_ce, lse_*         pinned (brute force with math.fsum, torch
                            cross_entropy, W=0 closed form, merge order)
  partial_sumsq, tile_lse   pinned (sum identities with the row results)
  swiglu_grad, rmsnorm_bwd, pinned (central finite differences in numpy,
  mlp_layer_bwd             torch float64 autograd, scale invariance of
                            RMSNorm: dh . h = 0 when eps = 0 and dy = 0)
The page's own numbers: the page prints none for this path, so nothing is
pinned to page values (parity unpinned against the page itself).
"""

from . import codecs  # noqa: F401
from .reference import (  # noqa: F401
    gemm_nt,
    residual_add,
    rms_scale,
    rmsnorm,
    silu,
    swiglu,
    mlp_block,
    swiglu_grad,
    rmsnorm_bwd,
    mlp_layer_bwd,
    fp8_mlp_block,
    fp8_h_amax,
    rope_tables,
    apply_rope,
    attn_in_block,
    attention_causal_gqa,
    layer_forward,
    logsumexp_rows,
    lm_head_ce,
    partial_sumsq,
    tile_lse,
    lse_merge,
)

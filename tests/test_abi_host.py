"""The C ABI without a GPU: the library loads, exports every function that
include/coda.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

from gemm_epilogue_transformer_gemm1_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coda.h")

ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_DEVICE = -1, -2, -3, -4, -5
A16 = 0x10000  # a fake 16-byte-aligned address, never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(coda_\w+)\s*\(", text,
                                 re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libcoda.so not built")
    return ops.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 17
    raw = ctypes.CDLL(ops.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
        assert n in ops._SIGNATURES, f"binding lacks {n}"


def test_version_status_and_tiles(L):
    assert L.coda_abi_version() >= 1
    for s in (0, -1, -2, -3, -4, -5, -6, -99):
        assert len(ops.status_string(s)) > 0
    w = L.coda_rms_tile_width()
    assert w in (64, 128, 256)
    assert L.coda_rms_tiles(2048) == 2048 // w
    assert L.coda_rms_tiles(2048 + 16) == 2048 // w + 1
    assert L.coda_rms_tiles(0) == 0
    v = L.coda_lse_tile_width()
    assert L.coda_lse_tiles(128256) == (128256 + v - 1) // v


def test_gemm1_validation(L):
    f = L.coda_gemm_residual_partialrms
    ok = dict(dtype=0, A=A16, W=A16, sa=None, sw=None, res=A16, h=A16, P=A16, s8=None,
              h8=None, am=None, M=64, N=256, K=256, st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["dtype"], a["A"], a["W"], a["sa"], a["sw"], a["res"], a["h"], a["P"],
                 a["s8"], a["h8"], a["am"], a["M"], a["N"], a["K"], a["st"])
    assert call(A=None) == ERR_NULL
    assert call(P=None) == ERR_NULL
    assert call(dtype=7) == ERR_DTYPE
    assert call(sa=A16) == ERR_DTYPE          # scales only belong to the fp8 form
    assert call(M=0) == ERR_SHAPE
    assert call(N=8) == ERR_SHAPE
    assert call(N=264) == ERR_SHAPE            # N % 16
    assert call(K=96) == ERR_SHAPE             # K % 64
    assert call(K=32) == ERR_SHAPE
    assert call(M=1 << 20, K=2048) == ERR_SHAPE  # element count limit
    assert call(A=A16 + 8) == ERR_ALIGN
    assert call(P=A16 + 2) == ERR_ALIGN


def test_other_validation(L):
    assert L.coda_rms_reduce(None, None, 2, 8, 8, 1e-5, A16, None, None, None) == ERR_NULL
    assert L.coda_rms_reduce(A16, None, 0, 8, 8, 1e-5, A16, None, None, None) == ERR_SHAPE
    assert L.coda_rms_reduce(A16, None, 2, 8, 8, -1.0, A16, None, None, None) == ERR_SHAPE
    assert L.coda_rms_reduce(A16, A16, 2, 8, 8, 1e-5, A16, None, None, None) == ERR_NULL
    f = L.coda_gemm_rowscale_swiglu
    assert f(0, A16, None, A16, None, None, None, A16, A16, 64, 64, 64, None) == ERR_NULL
    assert f(0, A16, None, A16, A16, None, None, A16, A16, 64, 65, 64, None) == ERR_SHAPE
    assert f(0, A16, A16, A16, A16, None, None, A16, A16, 64, 64, 64, None) == ERR_DTYPE
    assert f(0, A16, None, A16, A16 + 4, None, None, A16, A16, 64, 64, 64, None) == ERR_ALIGN
    assert L.coda_fold_gamma(A16, A16, A16, 4, 12, None) == ERR_SHAPE
    assert L.coda_gemm_bf16(A16, A16, None, 64, 64, 64, None) == ERR_NULL
    assert L.coda_residual_add(A16, A16, A16, 12, None) == ERR_SHAPE
    assert L.coda_rmsnorm(A16, A16, 1e-5, A16, 4, 32768, None) == ERR_SHAPE
    assert L.coda_swiglu(A16, A16 + 8, 4, 64, None) == ERR_ALIGN


@pytest.mark.skipif(torch.cuda.is_available(), reason="would launch on fake pointers")
def test_valid_arguments_without_gpu_report_device_error(L):
    # With every argument valid, the next step is the device check, which
    # fails cleanly on a machine without a gfx950 GPU.
    st = L.coda_gemm_bf16(A16, A16, A16, 64, 64, 64, None)
    assert st == ERR_DEVICE
    assert L.coda_gemm_bf16_splitk(A16, A16, A16, A16, 64, 64, 256, 4, None) == ERR_DEVICE


def test_backward_validation(L):
    # coda_gemm_rowscale_swiglu_save(X, Wg, Wu, r, out, gu, M, N, K, stream)
    s = L.coda_gemm_rowscale_swiglu_save
    assert s(A16, A16, A16, A16, A16, None, 64, 256, 256, None) == ERR_NULL
    assert s(A16, A16, A16, A16, A16, A16, 64, 264, 256, None) == ERR_SHAPE
    assert s(A16, A16, A16, A16, A16, A16 + 8, 64, 256, 256, None) == ERR_ALIGN
    assert s(A16, A16, A16, A16, A16, A16, 1 << 16, 1 << 14, 64, None) == ERR_SHAPE  # M x 2N
    # coda_gemm_swiglu_bwd(dY, WdT, gu, dz, partial_dot, M, N, K, stream)
    b = L.coda_gemm_swiglu_bwd
    assert b(A16, A16, A16, A16, None, 64, 256, 256, None) == ERR_NULL
    assert b(A16, A16, A16, A16, A16, 64, 256, 96, None) == ERR_SHAPE   # K % 64
    assert b(A16, A16, A16, A16, A16, 64, 8, 256, None) == ERR_SHAPE    # N >= 16
    assert b(A16, A16, A16 + 4, A16, A16, 64, 256, 256, None) == ERR_ALIGN
    assert b(A16, A16, A16, A16, A16 + 2, 64, 256, 256, None) == ERR_ALIGN
    # coda_rms_bwd_reduce(partial_dot, T, M, r, N, c, stream)
    c = L.coda_rms_bwd_reduce
    assert c(A16, 2, 8, None, 8, A16, None) == ERR_NULL
    assert c(A16, 0, 8, A16, 8, A16, None) == ERR_SHAPE
    assert c(A16, 2, 8, A16, 0, A16, None) == ERR_SHAPE
    assert c(A16, 2, 8, A16, 8, A16 + 2, None) == ERR_ALIGN
    # coda_gemm_rmsnorm_bwd(dz, W2T, h, dY, r, c, dh, M, N, K, stream)
    g = L.coda_gemm_rmsnorm_bwd
    assert g(A16, A16, A16, A16, A16, None, A16, 64, 256, 512, None) == ERR_NULL
    assert g(A16, A16, A16, A16, A16, A16, A16, 0, 256, 512, None) == ERR_SHAPE
    assert g(A16, A16, A16, A16, A16, A16, A16, 64, 256, 544, None) == ERR_SHAPE  # K % 64
    assert g(A16, A16, A16 + 8, A16, A16, A16, A16, 64, 256, 512, None) == ERR_ALIGN
    # unfused pieces and the transpose
    assert L.coda_swiglu_bwd(A16, None, A16, 64, 256, None) == ERR_NULL
    assert L.coda_swiglu_bwd(A16, A16, A16, 64, 12, None) == ERR_SHAPE
    assert L.coda_rmsnorm_bwd(A16, A16, A16, 1e-5, A16, 64, 32768, None) == ERR_SHAPE
    assert L.coda_rmsnorm_bwd(A16, A16, A16, -1.0, A16, 64, 256, None) == ERR_SHAPE
    assert L.coda_transpose_bf16(A16, None, 4, 8, None, 4, None) == ERR_NULL
    assert L.coda_transpose_bf16(A16, None, 4, 8, A16, 3, None) == ERR_SHAPE    # ld_dst < rows
    assert L.coda_transpose_bf16(A16 + 1, None, 4, 8, A16, 4, None) == ERR_ALIGN
    assert L.coda_transpose_bf16(A16, A16 + 2, 4, 8, A16, 4, None) == ERR_ALIGN
    # coda_gemm_bf16_splitk(A, W, C, workspace, M, N, K, parts, stream)
    k = L.coda_gemm_bf16_splitk
    assert k(A16, A16, A16, None, 64, 256, 512, 4, None) == ERR_NULL
    assert k(A16, A16, A16, A16, 64, 256, 512, 0, None) == ERR_SHAPE     # parts >= 1
    assert k(A16, A16, A16, A16, 64, 256, 512, 17, None) == ERR_SHAPE    # parts <= 16
    assert k(A16, A16, A16, A16, 64, 256, 384, 4, None) == ERR_SHAPE     # K % (64 parts)
    assert k(A16, A16, A16, A16, 64, 264, 512, 4, None) == ERR_SHAPE     # N % 16
    assert k(A16, A16, A16, A16, 256, 1 << 21, 64, 1, None) == ERR_SHAPE  # 256 N fp32 rows
    assert k(A16, A16, A16, A16 + 8, 64, 256, 512, 4, None) == ERR_ALIGN


def test_noalloc_lse_validation(L):
    """The LM head that allocates nothing rejects, before any HIP call, sizes
    whose partials exceed its static scratch, and the usual bad arguments."""
    f = L.coda_gemm_block_lse_noalloc
    assert L.coda_lse_noalloc_max_bytes() == 64 << 20
    # M = 16384 at V = 128256 needs 2 x 1002 x 16384 x 4 bytes: past 64 MiB
    assert f(A16, A16, None, A16, None, A16, 16384, 128256, 2048, None) == ERR_SHAPE
    assert f(None, A16, None, A16, None, A16, 64, 1024, 64, None) == ERR_NULL
    assert f(A16, A16, None, A16, None, A16, 64, 1000, 64, None) == ERR_SHAPE   # V % 16
    assert f(A16 + 2, A16, None, A16, None, A16, 64, 1024, 64, None) == ERR_ALIGN
    # the full LM-head size fits: validation passes and only the device check remains
    assert f(A16, A16, None, A16, None, A16, 8192, 128256, 2048, None) == ERR_DEVICE


def test_attention_validation(L):
    """coda_attention_fwd(qkv, o, M, seq_len, n_q, n_kv, head_dim, stream)
    rejects bad arguments before any HIP call."""
    f = L.coda_attention_fwd
    assert f(None, A16, 4096, 2048, 32, 8, 64, None) == ERR_NULL
    assert f(A16, None, 4096, 2048, 32, 8, 64, None) == ERR_NULL
    assert f(A16, A16, 4096, 2048, 32, 8, 96, None) == ERR_SHAPE     # head size 64 or 128
    assert f(A16, A16, 4096, 2048, 32, 8, 256, None) == ERR_SHAPE
    assert f(A16, A16, 4096, 2048, 32, 6, 64, None) == ERR_SHAPE     # n_q % n_kv
    assert f(A16, A16, 4096, 2048, 0, 8, 64, None) == ERR_SHAPE
    assert f(A16, A16, 4096, 2048, 32, 0, 64, None) == ERR_SHAPE
    assert f(A16, A16, 4096, 2000, 32, 8, 64, None) == ERR_SHAPE     # seq_len % 128
    assert f(A16, A16, 4096, 0, 32, 8, 64, None) == ERR_SHAPE
    assert f(A16, A16, 6144, 4096, 32, 8, 64, None) == ERR_SHAPE     # M % seq_len
    assert f(A16, A16, 1024, 2048, 32, 8, 64, None) == ERR_SHAPE     # M < seq_len
    assert f(A16, A16, 1 << 20, 2048, 64, 8, 64, None) == ERR_SHAPE  # element count limit
    assert f(A16 + 8, A16, 4096, 2048, 32, 8, 64, None) == ERR_ALIGN
    assert f(A16, A16 + 2, 4096, 2048, 32, 8, 64, None) == ERR_ALIGN
    if not torch.cuda.is_available():
        assert f(A16, A16, 8192, 2048, 32, 8, 64, None) == ERR_DEVICE
        assert f(A16, A16, 8192, 2048, 64, 8, 128, None) == ERR_DEVICE
    with pytest.raises(ValueError, match="shape"):   # o of another width
        ops.attention_fwd(torch.zeros(256, 6 * 64, dtype=torch.bfloat16),
                          torch.zeros(256, 3 * 64, dtype=torch.bfloat16), 128, 4, 1)


def test_rope_head_sizes(L):
    """The RoPE calls take heads of 64 or 128 and reject other sizes before
    any HIP call."""
    g = L.coda_gemm_rope
    # (h, Wqkv, r, cos, sin, pos, max_pos, qkv, M, K, n_q, n_kv, head_dim, stream)
    for hd in (32, 96, 256):
        assert g(A16, A16, A16, A16, A16, A16, 64, A16, 64, 64, 4, 2, hd, None) == ERR_SHAPE
        assert L.coda_rope_apply(A16, A16, A16, A16, 64, 64, 4, 2, hd, None) == ERR_SHAPE
    if not torch.cuda.is_available():
        for hd in (64, 128):
            assert g(A16, A16, A16, A16, A16, A16, 64, A16, 64, 64, 4, 2, hd, None) == ERR_DEVICE
            assert L.coda_rope_apply(A16, A16, A16, A16, 64, 64, 4, 2, hd, None) == ERR_DEVICE


def test_binding_checks_backward_shapes():
    """The Python binding refuses output tensors of the wrong shape before any
    call (CPU tensors are rejected for not being on the device, which needs
    no GPU to check)."""
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.gemm_swiglu_bwd(x, torch.zeros(16, 8, dtype=torch.bfloat16),
                            torch.zeros(4, 16, dtype=torch.bfloat16),
                            torch.zeros(4, 32, dtype=torch.bfloat16),
                            torch.zeros(1, 4, dtype=torch.float32))
    with pytest.raises(ValueError):
        ops.transpose(x, torch.zeros(8, 3, dtype=torch.bfloat16))


def test_binding_checks_forward_shapes(L):
    """Wrong-sized outputs or operands are refused on the host, before the
    kernels could index past a buffer (shape errors are raised before the
    device check, so CPU tensors suffice)."""
    bf, f32 = torch.bfloat16, torch.float32
    A, W = torch.zeros(64, 256, dtype=bf), torch.zeros(256, 256, dtype=bf)
    res, h = torch.zeros(64, 256, dtype=bf), torch.zeros(64, 256, dtype=bf)
    T = ops.rms_tiles(256)
    with pytest.raises(ValueError, match="shape"):   # partial sums too small
        ops.gemm_residual_partialrms(A, W, res, h, torch.zeros(T - 1, 64, dtype=f32))
    with pytest.raises(ValueError, match="shape"):   # h of another width
        ops.gemm_residual_partialrms(A, W, res, torch.zeros(64, 128, dtype=bf),
                                     torch.zeros(T, 64, dtype=f32))
    with pytest.raises(ValueError, match="shape"):   # r too short
        ops.rms_reduce(torch.zeros(T, 64, dtype=f32), 256, 1e-5, torch.zeros(32, dtype=f32))
    with pytest.raises(ValueError, match="shape"):   # out of the wrong width
        ops.gemm_rowscale_swiglu(A, W, W, torch.zeros(64, dtype=f32),
                                 torch.zeros(64, 512, dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        ops.gemm_bf16(A, W, torch.zeros(64, 255, dtype=bf))
    with pytest.raises(ValueError, match="shape"):   # LSE workspace for fewer tiles
        ops.gemm_block_lse(A, W, torch.zeros(64, dtype=torch.int32),
                           torch.zeros(1, 64, dtype=f32), torch.zeros(1, 64, dtype=f32),
                           torch.zeros(64, dtype=f32), torch.zeros(64, dtype=f32))
    with pytest.raises(ValueError, match="shape"):   # RoPE tables of another head size
        ops.gemm_rope(A, torch.zeros(6 * 64, 256, dtype=bf), torch.zeros(64, dtype=f32),
                      torch.zeros(16, 16, dtype=f32), torch.zeros(16, 16, dtype=f32),
                      torch.zeros(64, dtype=torch.int32), torch.zeros(64, 6 * 64, dtype=bf),
                      4, 1, 64)
    with pytest.raises(ValueError, match="shape"):
        ops.rmsnorm(h, torch.zeros(255, dtype=f32), 1e-5, h)
    with pytest.raises(ValueError, match="shape"):
        ops.swiglu(torch.zeros(64, 512, dtype=bf), torch.zeros(64, 512, dtype=bf))


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with a message
    (before touching torch or a device)."""
    import subprocess
    import sys
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert p.returncode == 2
    assert "one GPU" in p.stderr

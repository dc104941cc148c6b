"""Thin Python binding of libcoda's C ABI (include/coda.h).

Argument marshalling only: each function takes torch device tensors, checks
dtype / device / contiguity, and passes raw pointers plus the current torch
stream to the C entry point of the same name.  Every computation runs in the
library's HIP kernels; there is no fallback: if libcoda.so is missing or a
call fails, a RuntimeError is raised.

bf16 tensors are torch.bfloat16; e4m3 tensors are torch.uint8 (E4M3FN codes)
or torch.float8_e4m3fn.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoda.so")

CODA_BF16 = 0
CODA_FP8_E4M3 = 1

_lib = None

_c_int, _c_float, _c_double = ctypes.c_int, ctypes.c_float, ctypes.c_double
_p, _i64 = ctypes.c_void_p, ctypes.c_int64

_SIGNATURES = {
    "coda_abi_version": ([], _c_int),
    "coda_status_string": ([_c_int], ctypes.c_char_p),
    "coda_rms_tile_width": ([], _c_int),
    "coda_rms_tiles": ([_c_int], _c_int),
    "coda_lse_tile_width": ([], _c_int),
    "coda_lse_tiles": ([_c_int], _c_int),
    "coda_gemm_residual_partialrms": ([_c_int, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                       _c_int, _c_int, _c_int, _p], _c_int),
    "coda_rms_reduce": ([_p, _p, _c_int, _c_int, _c_int, _c_float, _p, _p, _p, _p], _c_int),
    "coda_gemm_rowscale_swiglu": ([_c_int, _p, _p, _p, _p, _p, _p, _p, _p, _c_int, _c_int,
                                   _c_int, _p], _c_int),
    "coda_gemm_rope": ([_p, _p, _p, _p, _p, _p, _c_int, _p, _c_int, _c_int, _c_int, _c_int,
                        _c_int, _p], _c_int),
    "coda_gemm_block_lse": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _p],
                            _c_int),
    "coda_fold_gamma": ([_p, _p, _p, _c_int, _c_int, _p], _c_int),
    "coda_rope_tables": ([_c_double, _c_int, _c_int, _p, _p, _p], _c_int),
    "coda_gemm_bf16": ([_p, _p, _p, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_gemm_bf16_splitk": ([_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_residual_add": ([_p, _p, _p, _i64, _p], _c_int),
    "coda_rmsnorm": ([_p, _p, _c_float, _p, _c_int, _c_int, _p], _c_int),
    "coda_swiglu": ([_p, _p, _c_int, _c_int, _p], _c_int),
    "coda_gemm_fp8": ([_p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_quantize_e4m3": ([_p, _i64, _p, _p, _p, _p, _p], _c_int),
    "coda_rope_apply": ([_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_cross_entropy_rows": ([_p, _p, _p, _p, _c_int, _c_int, _p], _c_int),
    "coda_gemm_rowscale_swiglu_save": ([_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _p],
                                       _c_int),
    "coda_gemm_swiglu_bwd": ([_p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_rms_bwd_reduce": ([_p, _c_int, _c_int, _p, _c_int, _p, _p], _c_int),
    "coda_gemm_rmsnorm_bwd": ([_p, _p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_swiglu_bwd": ([_p, _p, _p, _c_int, _c_int, _p], _c_int),
    "coda_transpose_bf16": ([_p, _p, _c_int, _c_int, _p, _c_int, _p], _c_int),
    "coda_rmsnorm_bwd": ([_p, _p, _p, _c_float, _p, _c_int, _c_int, _p], _c_int),
    "coda_dgamma_slices": ([_c_int], _c_int),
    "coda_attention_fwd": ([_p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_lse_noalloc_max_bytes": ([], ctypes.c_size_t),
    "coda_gemm_block_lse_noalloc": ([_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _p],
                                    _c_int),
    "coda_gemm_wgrad_gamma": ([_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _p], _c_int),
    "coda_dgamma_reduce": ([_p, _c_int, _c_int, _p, _p, _p], _c_int),
    "coda_col_dot_partial": ([_p, _p, _c_int, _c_int, _p, _p], _c_int),
}


class CodaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def lib():
    """Load libcoda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gemm_epilogue_transformer_gemm1_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def status_string(status):
    return lib().coda_status_string(status).decode()


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise CodaError(name, st)


def _ptr(t, dtype=None, what="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{what} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _shape(t, shape, what):
    """Host-side size check: the kernels index the buffers by the sizes passed
    through the C ABI, which cannot see a buffer's extent."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _want(t, shape, what):
    if t is not None:
        _shape(t, shape, what)


def _scalar(t, what):
    if t is not None and t.numel() < 1:
        raise ValueError(f"{what} must hold one value (shape {tuple(t.shape)})")


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


_BF16 = torch.bfloat16
_F32 = torch.float32
_I32 = torch.int32
_E4M3 = (torch.uint8, torch.float8_e4m3fn)


def rms_tile_width():
    return lib().coda_rms_tile_width()


def rms_tiles(N):
    return lib().coda_rms_tiles(N)


def lse_tile_width():
    return lib().coda_lse_tile_width()


def lse_tiles(V):
    return lib().coda_lse_tiles(V)


def gemm_residual_partialrms(A, W, residual, h, partial_sumsq, a_scale=None, w_scale=None,
                             h8_scale=None, h8=None, partial_amax=None, stream=None):
    """h = residual + A W^T (*scales); partial sums of squares of h per tile."""
    fp8 = A.dtype in _E4M3
    dt = CODA_FP8_E4M3 if fp8 else CODA_BF16
    M, K = A.shape
    N = W.shape[0]
    T = rms_tiles(N)
    for t, shp, what in ((W, (N, K), "W"), (residual, (M, N), "residual"), (h, (M, N), "h"),
                         (partial_sumsq, (T, M), "partial_sumsq"), (h8, (M, N), "h8"),
                         (partial_amax, (T, M), "partial_amax")):
        _want(t, shp, what)
    for t, what in ((a_scale, "a_scale"), (w_scale, "w_scale"), (h8_scale, "h8_scale")):
        _scalar(t, what)
    _call("coda_gemm_residual_partialrms", dt,
          _ptr(A, _E4M3 if fp8 else _BF16, "A"), _ptr(W, _E4M3 if fp8 else _BF16, "W"),
          _ptr(a_scale, _F32, "a_scale"), _ptr(w_scale, _F32, "w_scale"),
          _ptr(residual, _BF16, "residual"), _ptr(h, _BF16, "h"),
          _ptr(partial_sumsq, _F32, "partial_sumsq"), _ptr(h8_scale, _F32, "h8_scale"),
          _ptr(h8, _E4M3, "h8"), _ptr(partial_amax, _F32, "partial_amax"),
          M, N, K, _stream(stream))


def rms_reduce(partial_sumsq, N, eps, r, partial_amax=None, h_amax=None, h8_scale_out=None,
               stream=None):
    """r = 1/sqrt(sum_t partial / N + eps) per row (plus the fp8 amax)."""
    T, M = partial_sumsq.shape
    _shape(r, (M,), "r")
    _want(partial_amax, (T, M), "partial_amax")
    _scalar(h_amax, "h_amax")
    _scalar(h8_scale_out, "h8_scale_out")
    _call("coda_rms_reduce", _ptr(partial_sumsq, _F32, "partial_sumsq"),
          _ptr(partial_amax, _F32, "partial_amax"), T, M, N, float(eps), _ptr(r, _F32, "r"),
          _ptr(h_amax, _F32, "h_amax"), _ptr(h8_scale_out, _F32, "h8_scale_out"),
          _stream(stream))


def gemm_rowscale_swiglu(X, Wg, Wu, r, out, x_scale=None, wg_scale=None, wu_scale=None,
                         stream=None):
    """out = silu(r * X Wg^T) * (r * X Wu^T) (*scales)."""
    fp8 = X.dtype in _E4M3
    dt = CODA_FP8_E4M3 if fp8 else CODA_BF16
    M, K = X.shape
    N = Wg.shape[0]
    wt = _E4M3 if fp8 else _BF16
    for t, shp, what in ((Wg, (N, K), "Wg"), (Wu, (N, K), "Wu"), (r, (M,), "r"),
                         (out, (M, N), "out")):
        _shape(t, shp, what)
    for t, what in ((x_scale, "x_scale"), (wg_scale, "wg_scale"), (wu_scale, "wu_scale")):
        _scalar(t, what)
    _call("coda_gemm_rowscale_swiglu", dt, _ptr(X, wt, "X"), _ptr(x_scale, _F32, "x_scale"),
          _ptr(Wg, wt, "Wg"), _ptr(Wu, wt, "Wu"), _ptr(wg_scale, _F32, "wg_scale"),
          _ptr(wu_scale, _F32, "wu_scale"), _ptr(r, _F32, "r"), _ptr(out, _BF16, "out"),
          M, N, K, _stream(stream))


def gemm_rowscale_swiglu_save(X, Wg, Wu, r, out, gu, stream=None):
    """out = silu(g) * u with g = r * X Wg^T, u = r * X Wu^T, and gu = [g | u]
    kept for the backward pass (bf16)."""
    M, K = X.shape
    N = Wg.shape[0]
    for t, shp, what in ((Wg, (N, K), "Wg"), (Wu, (N, K), "Wu"), (r, (M,), "r"),
                         (out, (M, N), "out"), (gu, (M, 2 * N), "gu")):
        _shape(t, shp, what)
    _call("coda_gemm_rowscale_swiglu_save", _ptr(X, _BF16, "X"), _ptr(Wg, _BF16, "Wg"),
          _ptr(Wu, _BF16, "Wu"), _ptr(r, _F32, "r"), _ptr(out, _BF16, "out"),
          _ptr(gu, _BF16, "gu"), M, N, K, _stream(stream))


def gemm_swiglu_bwd(dY, WdT, gu, dz, partial_dot, stream=None):
    """dz = [dg | du] of SwiGLU given dout = dY WdT^T (never stored) and the
    saved gu = [g | u]; partial_dot[t, m] = sum over tile t of dg g + du u."""
    M, K = dY.shape
    N = WdT.shape[0]
    for t, shp, what in ((WdT, (N, K), "WdT"), (gu, (M, 2 * N), "gu"), (dz, (M, 2 * N), "dz"),
                         (partial_dot, (rms_tiles(N), M), "partial_dot")):
        _shape(t, shp, what)
    _call("coda_gemm_swiglu_bwd", _ptr(dY, _BF16, "dY"), _ptr(WdT, _BF16, "WdT"),
          _ptr(gu, _BF16, "gu"), _ptr(dz, _BF16, "dz"), _ptr(partial_dot, _F32, "partial_dot"),
          M, N, K, _stream(stream))


def rms_bwd_reduce(partial_dot, N, r, c, stream=None):
    """c[m] = r[m]^2 / N * sum_t partial_dot[t, m] (N = the normalised width)."""
    T, M = partial_dot.shape
    _shape(r, (M,), "r")
    _shape(c, (M,), "c")
    _call("coda_rms_bwd_reduce", _ptr(partial_dot, _F32, "partial_dot"), T, M, _ptr(r, _F32, "r"),
          int(N), _ptr(c, _F32, "c"), _stream(stream))


def dgamma_slices(M):
    """Number of 128-row slices of the dgamma partial sums for M weight rows."""
    return lib().coda_dgamma_slices(int(M))


def gemm_wgrad_gamma(A, B, W, gamma, dW, partial_dgamma, stream=None):
    """dW = bf16((A B^T) * gamma) with A = dz^T, B = (r h)^T, and the partial
    sums partial_dgamma[p, k] = sum over 128-row slice p of (A B^T)[n,k] W[n,k]."""
    M, K = A.shape
    N = B.shape[0]
    for t, shp, what in ((B, (N, K), "B"), (W, (M, N), "W"), (gamma, (N,), "gamma"),
                         (dW, (M, N), "dW"), (partial_dgamma, (dgamma_slices(M), N),
                                              "partial_dgamma")):
        _shape(t, shp, what)
    _call("coda_gemm_wgrad_gamma", _ptr(A, _BF16, "A"), _ptr(B, _BF16, "B"), _ptr(W, _BF16, "W"),
          _ptr(gamma, _F32, "gamma"), _ptr(dW, _BF16, "dW"),
          _ptr(partial_dgamma, _F32, "partial_dgamma"), M, N, K, _stream(stream))


def dgamma_reduce(partial, dgamma, gamma_div=None, stream=None):
    """dgamma[k] = sum_p partial[p, k] (divided by gamma_div[k] if given)."""
    P, N = partial.shape
    _shape(dgamma, (N,), "dgamma")
    gd = None
    if gamma_div is not None:
        _shape(gamma_div, (N,), "gamma_div")
        gd = _ptr(gamma_div, _F32, "gamma_div")
    _call("coda_dgamma_reduce", _ptr(partial, _F32, "partial"), P, N, gd,
          _ptr(dgamma, _F32, "dgamma"), _stream(stream))


def col_dot_partial(X, Y, partial, stream=None):
    """partial[p, k] = sum over 128-row slice p of X[n,k] Y[n,k] (bf16 inputs)."""
    M, N = X.shape
    _shape(Y, (M, N), "Y")
    _shape(partial, (dgamma_slices(M), N), "partial")
    _call("coda_col_dot_partial", _ptr(X, _BF16, "X"), _ptr(Y, _BF16, "Y"), M, N,
          _ptr(partial, _F32, "partial"), _stream(stream))


def gemm_rmsnorm_bwd(dz, W2T, h, dY, r, c, dh, stream=None):
    """dh = r * (dz W2T^T) - c * h + dY."""
    M, K = dz.shape
    N = W2T.shape[0]
    for t, shp, what in ((W2T, (N, K), "W2T"), (h, (M, N), "h"), (dY, (M, N), "dY"),
                         (r, (M,), "r"), (c, (M,), "c"), (dh, (M, N), "dh")):
        _shape(t, shp, what)
    _call("coda_gemm_rmsnorm_bwd", _ptr(dz, _BF16, "dz"), _ptr(W2T, _BF16, "W2T"),
          _ptr(h, _BF16, "h"), _ptr(dY, _BF16, "dY"), _ptr(r, _F32, "r"), _ptr(c, _F32, "c"),
          _ptr(dh, _BF16, "dh"), M, N, K, _stream(stream))


def transpose(src, dst, row_scale=None, stream=None):
    """dst[:, :rows] = src^T for src [rows, cols] (bf16), each source row
    scaled by row_scale[row] first if given; dst [cols, ld] may be a column
    slice of a wider row-major matrix (its row stride is ld)."""
    rows, cols = src.shape
    _want(row_scale, (rows,), "row_scale")
    if dst.dim() != 2 or dst.shape[0] != cols or dst.shape[1] < rows or dst.stride(1) != 1:
        raise ValueError(f"dst {tuple(dst.shape)} cannot hold the transpose of {tuple(src.shape)}")
    if dst.dtype != _BF16 or not dst.is_cuda:
        raise TypeError("dst must be a bf16 device tensor")
    ld = dst.stride(0)
    if ld < rows or dst.storage_offset() + (cols - 1) * ld + rows > dst.untyped_storage().nbytes() // 2:
        raise ValueError("dst's storage is too small for the transpose")
    _call("coda_transpose_bf16", _ptr(src, _BF16, "src"), _ptr(row_scale, _F32, "row_scale"),
          rows, cols, dst.data_ptr(), ld, _stream(stream))


def swiglu_bwd(dout, gu, dz, stream=None):
    """Unfused SwiGLU backward from a stored dout [M, N]."""
    M, N = dout.shape
    _shape(gu, (M, 2 * N), "gu")
    _shape(dz, (M, 2 * N), "dz")
    _call("coda_swiglu_bwd", _ptr(dout, _BF16, "dout"), _ptr(gu, _BF16, "gu"),
          _ptr(dz, _BF16, "dz"), M, N, _stream(stream))


def rmsnorm_bwd(G, h, dY, eps, dh, stream=None):
    """Unfused RMSNorm backward from a stored G = dz W' [M, N] (the row scale
    is recomputed from h)."""
    M, N = G.shape
    for t, shp, what in ((h, (M, N), "h"), (dY, (M, N), "dY"), (dh, (M, N), "dh")):
        _shape(t, shp, what)
    _call("coda_rmsnorm_bwd", _ptr(G, _BF16, "G"), _ptr(h, _BF16, "h"), _ptr(dY, _BF16, "dY"),
          float(eps), _ptr(dh, _BF16, "dh"), M, N, _stream(stream))


def gemm_rope(h, Wqkv, r, rope_cos, rope_sin, pos, qkv, n_q_heads, n_kv_heads, head_dim,
              stream=None):
    """qkv = RoPE(r * h Wqkv^T) on the q and k heads."""
    M, K = h.shape
    Nq = (n_q_heads + 2 * n_kv_heads) * head_dim
    _check_rope(rope_cos, rope_sin, head_dim)
    for t, shp, what in ((Wqkv, (Nq, K), "Wqkv"), (r, (M,), "r"), (pos, (M,), "pos"),
                         (qkv, (M, Nq), "qkv")):
        _shape(t, shp, what)
    _call("coda_gemm_rope", _ptr(h, _BF16, "h"), _ptr(Wqkv, _BF16, "Wqkv"), _ptr(r, _F32, "r"),
          _ptr(rope_cos, _F32, "rope_cos"), _ptr(rope_sin, _F32, "rope_sin"),
          _ptr(pos, _I32, "pos"), rope_cos.shape[0], _ptr(qkv, _BF16, "qkv"), M, K,
          n_q_heads, n_kv_heads, head_dim, _stream(stream))


def gemm_block_lse(X, W, labels, tile_max, tile_sumexp, label_logit, loss, lse=None, r=None,
                   stream=None):
    """Per-row cross entropy of z = (r *) X W^T without storing z."""
    M, K = X.shape
    V = W.shape[0]
    T = lse_tiles(V)
    for t, shp, what in ((W, (V, K), "W"), (labels, (M,), "labels"), (tile_max, (T, M), "tile_max"),
                         (tile_sumexp, (T, M), "tile_sumexp"), (label_logit, (M,), "label_logit"),
                         (loss, (M,), "loss"), (lse, (M,), "lse"), (r, (M,), "r")):
        _want(t, shp, what)
    _call("coda_gemm_block_lse", _ptr(X, _BF16, "X"), _ptr(W, _BF16, "W"), _ptr(r, _F32, "r"),
          _ptr(labels, _I32, "labels"), _ptr(tile_max, _F32, "tile_max"),
          _ptr(tile_sumexp, _F32, "tile_sumexp"), _ptr(label_logit, _F32, "label_logit"),
          _ptr(lse, _F32, "lse"), _ptr(loss, _F32, "loss"), M, V, K, _stream(stream))


def attention_fwd(qkv, o, seq_len, n_q_heads, n_kv_heads, head_dim=64, stream=None):
    """Causal grouped-query attention over sequences of seq_len rows of qkv
    (q | k | v) into o [M, n_q_heads * head_dim]."""
    M = qkv.shape[0]
    _shape(qkv, (M, (n_q_heads + 2 * n_kv_heads) * head_dim), "qkv")
    _shape(o, (M, n_q_heads * head_dim), "o")
    _call("coda_attention_fwd", _ptr(qkv, _BF16, "qkv"), _ptr(o, _BF16, "o"), M, int(seq_len),
          int(n_q_heads), int(n_kv_heads), int(head_dim), _stream(stream))


def gemm_block_lse_noalloc(X, W, labels, loss, lse=None, r=None, stream=None):
    """coda_gemm_block_lse with the partials in the library's static scratch
    (no allocation; calls on one GPU must not overlap)."""
    M, K = X.shape
    V = W.shape[0]
    _shape(W, (V, K), "W")
    for t, shp, what in ((labels, (M,), "labels"), (loss, (M,), "loss"), (lse, (M,), "lse"),
                         (r, (M,), "r")):
        _want(t, shp, what)
    _call("coda_gemm_block_lse_noalloc", _ptr(X, _BF16, "X"), _ptr(W, _BF16, "W"),
          _ptr(r, _F32, "r"), _ptr(labels, _I32, "labels"), _ptr(lse, _F32, "lse"),
          _ptr(loss, _F32, "loss"), M, V, K, _stream(stream))


def lse_noalloc_max_bytes():
    return int(lib().coda_lse_noalloc_max_bytes())


def fold_gamma(W, gamma, W_out, stream=None):
    N, K = W.shape
    _shape(gamma, (K,), "gamma")
    _shape(W_out, (N, K), "W_out")
    _call("coda_fold_gamma", _ptr(W, _BF16, "W"), _ptr(gamma, _F32, "gamma"),
          _ptr(W_out, _BF16, "W_out"), N, K, _stream(stream))


def _check_rope(rope_cos, rope_sin, head_dim):
    if rope_cos.dim() != 2 or rope_cos.shape[1] != head_dim // 2:
        raise ValueError(f"rope_cos has shape {tuple(rope_cos.shape)}, expected [max_pos, {head_dim // 2}]")
    _shape(rope_sin, rope_cos.shape, "rope_sin")


def rope_tables(theta, max_pos, head_dim, rope_cos, rope_sin, stream=None):
    _shape(rope_cos, (max_pos, head_dim // 2), "rope_cos")
    _shape(rope_sin, (max_pos, head_dim // 2), "rope_sin")
    _call("coda_rope_tables", float(theta), max_pos, head_dim, _ptr(rope_cos, _F32, "rope_cos"),
          _ptr(rope_sin, _F32, "rope_sin"), _stream(stream))


def gemm_bf16(A, W, C, stream=None):
    M, K = A.shape
    N = W.shape[0]
    _shape(W, (N, K), "W")
    _shape(C, (M, N), "C")
    _call("coda_gemm_bf16", _ptr(A, _BF16, "A"), _ptr(W, _BF16, "W"), _ptr(C, _BF16, "C"),
          M, N, K, _stream(stream))


def gemm_bf16_splitk(A, W, C, workspace, stream=None):
    """C = bf16(A W^T) with the reduction split in workspace.shape[0] parts
    (fp32 partial products in workspace [parts, M, N], summed in part order)."""
    M, K = A.shape
    N = W.shape[0]
    parts = workspace.shape[0]
    _shape(W, (N, K), "W")
    _shape(C, (M, N), "C")
    _shape(workspace, (parts, M, N), "workspace")
    _call("coda_gemm_bf16_splitk", _ptr(A, _BF16, "A"), _ptr(W, _BF16, "W"), _ptr(C, _BF16, "C"),
          _ptr(workspace, _F32, "workspace"), M, N, K, parts, _stream(stream))


def residual_add(y, res, h, stream=None):
    _shape(res, y.shape, "res")
    _shape(h, y.shape, "h")
    _call("coda_residual_add", _ptr(y, _BF16, "y"), _ptr(res, _BF16, "res"), _ptr(h, _BF16, "h"),
          y.numel(), _stream(stream))


def rmsnorm(h, gamma, eps, out, stream=None):
    M, N = h.shape
    _shape(gamma, (N,), "gamma")
    _shape(out, (M, N), "out")
    _call("coda_rmsnorm", _ptr(h, _BF16, "h"), _ptr(gamma, _F32, "gamma"), float(eps),
          _ptr(out, _BF16, "out"), M, N, _stream(stream))


def swiglu(gu, out, stream=None):
    M, N2 = gu.shape
    if N2 % 2:
        raise ValueError(f"gu has an odd width {N2}")
    _shape(out, (M, N2 // 2), "out")
    _call("coda_swiglu", _ptr(gu, _BF16, "gu"), _ptr(out, _BF16, "out"), M, N2 // 2,
          _stream(stream))


def rope_apply(qkv, rope_cos, rope_sin, pos, n_q_heads, n_kv_heads, head_dim, stream=None):
    """In-place RoPE on the q and k heads of a stored qkv (unfused baseline)."""
    M = qkv.shape[0]
    _check_rope(rope_cos, rope_sin, head_dim)
    _shape(qkv, (M, (n_q_heads + 2 * n_kv_heads) * head_dim), "qkv")
    _shape(pos, (M,), "pos")
    _call("coda_rope_apply", _ptr(qkv, _BF16, "qkv"), _ptr(rope_cos, _F32, "rope_cos"),
          _ptr(rope_sin, _F32, "rope_sin"), _ptr(pos, _I32, "pos"), rope_cos.shape[0], M,
          n_q_heads, n_kv_heads, head_dim, _stream(stream))


def cross_entropy_rows(logits, labels, lse, loss, stream=None):
    """Per-row cross entropy of stored bf16 logits (unfused baseline)."""
    M, V = logits.shape
    for t, shp, what in ((labels, (M,), "labels"), (lse, (M,), "lse"), (loss, (M,), "loss")):
        _shape(t, shp, what)
    _call("coda_cross_entropy_rows", _ptr(logits, _BF16, "logits"), _ptr(labels, _I32, "labels"),
          _ptr(lse, _F32, "lse"), _ptr(loss, _F32, "loss"), M, V, _stream(stream))


def gemm_fp8(A, W, a_scale, w_scale, C, stream=None):
    """C = bf16(A W^T * a_scale * w_scale), e4m3 operands (unfused baseline).
    C may be a column slice of a wider row-major buffer (its row stride is used)."""
    M, K = A.shape
    N = W.shape[0]
    _shape(W, (N, K), "W")
    _scalar(a_scale, "a_scale")
    _scalar(w_scale, "w_scale")
    if C.stride(1) != 1 or C.shape != (M, N):
        raise ValueError("C must be [M, N] with unit column stride")
    if not C.is_cuda or C.dtype != _BF16:
        raise TypeError("C must be a bf16 device tensor")
    _call("coda_gemm_fp8", _ptr(A, _E4M3, "A"), _ptr(W, _E4M3, "W"), _ptr(a_scale, _F32, "a_scale"),
          _ptr(w_scale, _F32, "w_scale"), C.data_ptr(), C.stride(0), M, N, K, _stream(stream))


def quantize_e4m3(x, s_in, out, amax, s_out, stream=None):
    """out = e4m3(x / s_in), amax = max|x|, s_out = amax / 448 (unfused baseline)."""
    if out.numel() != x.numel():
        raise ValueError(f"out holds {out.numel()} values, x {x.numel()}")
    for t, what in ((s_in, "s_in"), (amax, "amax"), (s_out, "s_out")):
        _scalar(t, what)
    _call("coda_quantize_e4m3", _ptr(x, _BF16, "x"), x.numel(), _ptr(s_in, _F32, "s_in"),
          _ptr(out, _E4M3, "out"), _ptr(amax, _F32, "amax"), _ptr(s_out, _F32, "s_out"),
          _stream(stream))

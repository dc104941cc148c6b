"""Helpers for the GPU tests: host <-> device conversion and error metrics.
Runs the HIP path only through the C ABI binding (gemm_epilogue_transformer_gemm1_amd.ops)."""
import sys

import numpy as np
import torch

from gemm_epilogue_transformer_gemm1_amd import ops
from oracle import codecs

DEV = "cuda:0"

# Tolerances fixed by the accuracy requirement of the hot path:
TOL_BF16 = 1e-2   # max|err| / max|ref| for bf16 outputs
TOL_FP8 = 5e-2    # the same for outputs of the fp8 path
TOL_ROW = 1e-4    # relative error per row for r and for the per-row loss


def say(msg):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def bf16_encode_few(x):
    """The oracle's bf16 encoder applied to each distinct value of `x` and
    mapped back: the same bits, fast for large arrays of few values (the
    integer-exact tests)."""
    vals, inv = np.unique(np.asarray(x, dtype=np.float64), return_inverse=True)
    return codecs.bf16_encode(vals)[inv].reshape(np.shape(x))


def bf16_host(t):
    """torch.bfloat16 device tensor -> float64 numpy (via the oracle's decoder)."""
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return codecs.bf16_decode(bits)


def f32_host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def dec_bf16(bits):
    return codecs.bf16_decode(bits)


def norm_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def row_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)))


def sample_rows(M, n=48, seed=0):
    """Rows to check at full size: first, last, tile edges and random ones."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, 15, 16, 127, 128, 255, 256, M // 2, M - 257, M - 256, M - 2, M - 1]
    rows = set(r for r in edges if 0 <= r < M)
    rows.update(int(x) for x in rng.integers(0, M, size=n))
    return np.array(sorted(rows))


class MaxErr:
    """max|err| / max|ref| of a whole tensor accumulated over row chunks."""

    def __init__(self):
        self.err = 0.0
        self.ref = 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        self.err = max(self.err, float(np.max(np.abs(got - ref))))
        self.ref = max(self.ref, float(np.max(np.abs(ref))))

    def value(self):
        return self.err / max(self.ref, 1e-300)


def row_chunks(M, chunk=2048):
    """Consecutive row ranges covering [0, M), for oracle runs over every row."""
    return [np.arange(m0, min(M, m0 + chunk)) for m0 in range(0, M, chunk)]

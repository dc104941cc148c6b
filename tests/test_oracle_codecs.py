"""The oracle's number-format codecs against the formats' definitions and
against torch's CPU casts (a library routine)."""
import numpy as np
import pytest
import torch

from oracle import codecs


def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_vs_torch():
    ours = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2  # 0x7F and 0xFF


def test_e4m3_known_values():
    # from the format definition: bias 7, 3 mantissa bits, no infinities
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in table.items():
        assert codecs.e4m3_decode(np.array([c], dtype=np.uint8))[0] == v, hex(c)


def test_e4m3_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = codecs.e4m3_decode(codes)
    back = codecs.e4m3_encode(vals)
    # -0 encodes to 0x80 and 0 to 0x00, so the round trip is exact on all finite codes
    assert np.array_equal(back, codes)
    assert np.array_equal(codecs.e4m3_encode_fast(vals), codes)
    # midpoints between neighbouring positive codes round to the even code
    pos = [c for c in range(0, 0x7F)]
    for c in pos[:-1]:
        a, b = codecs.e4m3_decode(np.array([c, c + 1], dtype=np.uint8))
        mid = (a + b) / 2
        want = c if c % 2 == 0 else c + 1
        assert codecs.e4m3_encode(np.array([mid]))[0] == want, hex(c)
        assert codecs.e4m3_encode_fast(np.array([mid]))[0] == want, hex(c)
        assert codecs.e4m3_encode(np.array([-mid]))[0] == (want | 0x80)


def test_e4m3_saturates():
    x = np.array([448.0, 449.0, 464.0, 500.0, 1e30, -1e9, -448.5])
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert list(codecs.e4m3_encode(x)) == want
    assert list(codecs.e4m3_encode_fast(x)) == want


def test_e4m3_encode_vs_torch_random():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 300)])
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3_encode_fast(x), ref)
    assert np.array_equal(codecs.e4m3_encode(x[:3000]), ref[:3000])


def test_bf16_decode_vs_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_vs_torch():
    rng = np.random.default_rng(1)
    # float32-exact inputs (torch rounds float32 -> bf16 once, so no double rounding)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    # ties: bf16 value + half a bf16 ulp, exactly representable in float32
    base = torch.from_numpy(x[:500]).to(torch.bfloat16).to(torch.float32).numpy()
    ulp = np.abs(base) * 2.0 ** -8
    ties = (base + np.sign(base) * ulp / 2).astype(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-40, 3e38], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_encode(x.astype(np.float64)), ref)

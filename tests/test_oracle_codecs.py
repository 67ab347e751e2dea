"""Pins of the oracle's storage codecs and FP8 quantiser.

Each check compares the oracle with something other than itself: torch's own
dtype reinterpretation (a library routine), values fixed by the formats'
definitions, and exhaustive enumeration.
"""

import numpy as np
import pytest
import torch

from oracle import codecs


def test_fp16_decode_exhaustive_vs_torch():
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.float16).double().numpy()
    got = codecs.decode(codes, codecs.F16)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(got[m]))


def test_bf16_decode_exhaustive_vs_torch():
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = codecs.decode(codes, codecs.BF16)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(got[m]))


def test_f32_decode_sample_vs_torch():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    ref = torch.from_numpy(codes.view(np.int32)).view(torch.float32).double().numpy()
    got = codecs.decode(codes, codecs.F32)
    m = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(ref[m], got[m])


def test_e4m3_table_vs_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = codecs.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(got[m]))


def test_e4m3_definition_anchors():
    # values fixed by the E4M3FN definition
    t = codecs.E4M3_TABLE
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0                  # exponent field 7 = bias
    assert t[0x7E] == 448.0                # largest finite
    assert t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    # finite codes are strictly increasing in magnitude on 0x00..0x7E
    assert np.all(np.diff(t[:0x7F]) > 0)


@pytest.mark.parametrize("scale", [1.0, 0.0131, 2.0 ** -5, 3.7])
def test_quantizer_exhaustive_bf16_inputs_vs_torch(scale):
    """Every bf16 input, clamped then cast by torch (RNE, saturation by the
    explicit clamp), must match the oracle's quantiser bit for bit."""
    codes = np.arange(65536, dtype=np.uint16)
    x = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float()
    y = x / torch.tensor(np.float32(scale))            # fp32 division
    finite = torch.isfinite(y) | torch.isinf(y)
    ref = y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.quantize_e4m3(x.numpy(), scale)
    f = finite.numpy()
    assert np.array_equal(ref[f], got[f])
    nan_in = ~f
    assert np.all(np.isnan(codecs.E4M3_TABLE[got[nan_in]]))


def test_quantizer_exhaustive_f16_inputs_vs_torch():
    codes = np.arange(65536, dtype=np.uint16)
    x = torch.from_numpy(codes.view(np.int16)).view(torch.float16).float()
    scale = np.float32(0.25)
    y = x / torch.tensor(scale)
    ok = ~torch.isnan(y)
    ref = y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.quantize_e4m3(x.numpy(), float(scale))
    assert np.array_equal(ref[ok.numpy()], got[ok.numpy()])


def test_quantizer_ties_and_edges():
    q = lambda v: int(codecs.quantize_e4m3(np.array([v], np.float32), 1.0)[0])
    val = lambda c: codecs.E4M3_TABLE[c]
    assert val(q(1.0625)) == 1.0        # halfway between 1.0 and 1.125 -> even
    assert val(q(1.1875)) == 1.25       # halfway between 1.125 and 1.25 -> even
    assert val(q(464.0)) == 448.0       # clamped, never NaN
    assert val(q(1e30)) == 448.0
    assert val(q(-np.inf)) == -448.0
    assert val(q(2.0 ** -10)) == 0.0    # halfway between 0 and 2^-9 -> even (0)
    assert val(q(3 * 2.0 ** -10)) == 2 * 2.0 ** -9
    assert q(-0.0) == 0x80              # negative zero keeps its sign
    assert q(0.0) == 0x00
    assert q(np.nan) == 0x7F
    assert q(-np.float32(np.nan)) == 0xFF
    # every finite code is a fixed point of quantisation
    finite = np.array([c for c in range(256) if not np.isnan(val(c))])
    back = codecs.quantize_e4m3(codecs.E4M3_TABLE[finite].astype(np.float32), 1.0)
    assert np.array_equal(back, finite.astype(np.uint8))


def test_quantizer_divides_in_fp32():
    # x / s in fp32 differs from the fp64 quotient rounded once; the write
    # rule is the fp32 quotient. Pick x, s where rounding the quotient to fp32
    # moves it across an E4M3 rounding boundary.
    rng = np.random.default_rng(7)
    x = rng.standard_normal(100000).astype(np.float32)
    s = np.float32(0.0137)
    y32 = (x / s).astype(np.float64)
    got = codecs.E4M3_TABLE[codecs.quantize_e4m3(x, float(s))]
    ref = torch.from_numpy(y32).float().clamp(-448, 448).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, ref)


def test_encode_for_store_same_dtype_is_identity():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 65536, size=1000).astype(np.uint16)
    assert np.array_equal(codecs.encode_for_store(c, codecs.BF16, codecs.BF16), c)
    with pytest.raises(ValueError):
        codecs.encode_for_store(c, codecs.BF16, codecs.F16)

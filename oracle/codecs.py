"""Storage codes <-> exact float64 values (oracle; test infrastructure only).

The pages fix no storage format beyond "FP16" / "bf16" / "FP8 KV cache"
("Efficient Memory Management for Large Language Model Serving with
PagedAttention", per-token size paragraph: 2 bytes per FP16 element;
"Continuous Batching and PagedAttention", section "Sizing the KV cache for the
running 70B model": bf16; "KV Cache Preemption in vLLM", section "How much KV
cache a token costs": an FP8 KV cache halves the bytes per token). The
readings used here:

* fp32, fp16: IEEE-754 binary32 / binary16.
* bf16: the upper 16 bits of a binary32.
* FP8: OCP E4M3FN — sign, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 holds subnormals m * 2^-9; the all-ones code S.1111.111 is
  NaN; there is no infinity, so the largest finite magnitude is 448.
  A stored code means ``code_value * scale`` with one fp32 scale per tensor.

Every decode here is exact: each of these values is a float64.
"""

import numpy as np

F32 = "f32"
F16 = "f16"
BF16 = "bf16"
FP8 = "fp8_e4m3"

DTYPES = (F32, F16, BF16, FP8)

#: numpy unsigned type holding one storage code of each dtype
CODE_TYPE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16, FP8: np.uint8}

#: bytes per element
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, FP8: 1}

#: a NaN code of each dtype, used to poison memory that must never be read
NAN_CODE = {F32: 0x7FC00000, F16: 0x7E00, BF16: 0x7FC0, FP8: 0x7F}

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN code, straight from the field definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * man_field * 2.0 ** -9          # subnormal: m * 2^(1-7) / 8
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


#: the 256 E4M3FN values, index = code
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode(codes, dtype: str) -> np.ndarray:
    """Storage codes -> float64 values (exact)."""
    codes = np.asarray(codes, dtype=CODE_TYPE[dtype])
    if dtype == F32:
        return codes.view(np.float32).astype(np.float64)
    if dtype == F16:
        return codes.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (codes.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == FP8:
        return E4M3_TABLE[codes]
    raise ValueError(f"unknown dtype {dtype!r}")


def _round_half_even(x: np.ndarray) -> np.ndarray:
    # numpy's rint rounds halfway cases to the even neighbour
    return np.rint(x)


def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Round finite float64 magnitudes |y| <= 448 to the nearest E4M3 value,
    ties to even. Works on magnitudes (y >= 0)."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    sub = y < 2.0 ** -6                     # below the smallest normal: grid 2^-9
    out[sub] = _round_half_even(y[sub] * 2.0 ** 9) * 2.0 ** -9
    nrm = ~sub
    if np.any(nrm):
        # y = f * 2^e2 with f in [0.5, 1): the binade is [2^(e2-1), 2^e2) and
        # holds 8 values spaced 2^(e2-1-3).
        _, e2 = np.frexp(y[nrm])
        quantum = np.ldexp(1.0, e2 - 4)
        out[nrm] = _round_half_even(y[nrm] / quantum) * quantum
    return out


def e4m3_code_of_value(mag: np.ndarray, negative: np.ndarray) -> np.ndarray:
    """Exact E4M3 values (magnitudes on the grid, <= 448) -> codes."""
    mag = np.asarray(mag, dtype=np.float64)
    code = np.zeros(mag.shape, dtype=np.uint8)
    sub = mag < 2.0 ** -6
    code[sub] = (mag[sub] * 2.0 ** 9).astype(np.uint8)             # m, exponent 0
    nrm = ~sub
    if np.any(nrm):
        f, e2 = np.frexp(mag[nrm])                                  # f in [0.5, 1)
        exp_field = (e2 - 1) + 7
        man_field = (f * 16.0 - 8.0)                                # (2f - 1) * 8
        code[nrm] = (exp_field * 8 + man_field).astype(np.uint8)
    code |= np.where(negative, np.uint8(0x80), np.uint8(0))
    return code


def quantize_e4m3(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """FP8 quantiser of a slot write: code = RNE_e4m3(clamp(x / scale, +-448)).

    The division is one IEEE binary32 division (correctly rounded); NaN maps
    to the NaN code carrying the input's sign bit; -0 keeps its sign.
    """
    x32 = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y32 = x32 / np.float32(scale)             # binary32 division, RNE
    negative = np.signbit(y32)
    is_nan = np.isnan(y32)
    mag = np.abs(y32.astype(np.float64))
    mag = np.where(is_nan, 0.0, np.minimum(mag, E4M3_MAX))
    code = e4m3_code_of_value(e4m3_round(mag), negative)
    code = np.where(is_nan, np.where(negative, np.uint8(0xFF), np.uint8(0x7F)), code)
    return code.astype(np.uint8)


def encode_for_store(src_codes: np.ndarray, src_dtype: str, dst_dtype: str,
                     scale: float = 1.0) -> np.ndarray:
    """Codes a slot write stores for source codes of ``src_dtype``.

    Same dtype: the code is stored unchanged. FP8 destination: the source is
    first widened to binary32 (exact for fp32/fp16/bf16) and quantised.
    """
    if src_dtype == dst_dtype:
        return np.asarray(src_codes, dtype=CODE_TYPE[dst_dtype]).copy()
    if dst_dtype != FP8:
        raise ValueError(f"cannot store {src_dtype} into a {dst_dtype} pool")
    if src_dtype == FP8:
        raise ValueError("fp8 source needs an fp8 pool")
    x32 = decode(src_codes, src_dtype).astype(np.float32)          # exact widening
    return quantize_e4m3(x32, scale)

"""FP8 (e4m3) expert weights: decoding and per-row dequantization (oracle side).

Test infrastructure: only the tests, the package's smoke check and the bench's
CPU-baseline leg use this module; the GPU library never imports or links it.

The pages name FP8 and NVFP4 checkpoints of the model ("Google open-sources
DiffusionGemma: H100 reaches 1000 TPS", section "Hardware requirements";
"DiffusionGemma hits ~1,500 TPS on one H100", section "Serve it with vLLM") but
not their layout.  Format taken (a stated reading): each routed expert matrix
holds one byte per weight in the OCP FP8 E4M3 encoding (1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent 0 is subnormal, m x 2^-9; the
all-ones exponent and mantissa pattern is NaN; no infinities; largest finite
value 448) and one float32 scale per output row: W[n, k] = scale[n] * e4m3(code[n, k]).
"""
import numpy as np

E4M3_MAX = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """float64 value of every E4M3 code (uint8 array of any shape)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m, -9)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, v)


def dequantize_rows(codes, scales) -> np.ndarray:
    """W = scale[..., n, None] * e4m3(code[..., n, :]) in float64 (exact: a 4-bit
    significand times a float32 scale fits a double)."""
    return decode_e4m3(codes) * np.asarray(scales, dtype=np.float64)[..., None]

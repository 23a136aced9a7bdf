"""FP8 (e4m3) and MXFP4 expert weights: decoding and dequantization (oracle side).

Test infrastructure: only the tests, the package's smoke check and the bench's
CPU-baseline leg use this module; the GPU library never imports or links it.

The pages name FP8 and NVFP4 checkpoints of the model ("DiffusionGemma hits
~1,500 TPS on one H100", section "Serve it with vLLM") and a quantized model
that fits in about 18 GB ("Google open-sources DiffusionGemma: H100 reaches 1000
TPS", section "26B MoE Architecture, but Only 3.8B Activated") but not their
layout.  Format taken (a stated reading): each routed expert matrix
holds one byte per weight in the OCP FP8 E4M3 encoding (1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent 0 is subnormal, m x 2^-9; the
all-ones exponent and mantissa pattern is NaN; no infinities; largest finite
value 448) and one float32 scale per output row: W[n, k] = scale[n] * e4m3(code[n, k]).

MXFP4 (the OCP Microscaling Formats specification's FP4 type, CDNA4's native
4-bit format; the pages' NVFP4 is not built): each weight is an E2M1 code (1
sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent 0 is
subnormal, m x 2^-1; no infinities or NaN), two codes per byte with the lower
reduction index in the low nibble, and every 32 consecutive weights of a row
share one E8M0 scale byte s (an unsigned power of two, 2^(s - 127); 255 is NaN):
W[n, k] = 2^(s[n, k // 32] - 127) * e2m1(code[n, k]).
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


MX_BLOCK = 32
E2M1_MAX = 6.0


def decode_e2m1(nibbles) -> np.ndarray:
    """float64 value of every E2M1 code (integer array of values 0 .. 15)."""
    b = np.asarray(nibbles).astype(np.int64)
    if b.size and (b.min() < 0 or b.max() > 15):
        raise ValueError("E2M1 codes are 4-bit")
    sign = np.where(b >> 3, -1.0, 1.0)
    e = (b >> 1) & 0x3
    m = (b & 0x1).astype(np.float64)
    normal = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64))
    sub = m / 2.0
    return sign * np.where(e == 0, sub, normal)


def decode_e8m0(scale_bytes) -> np.ndarray:
    """float64 value 2^(s - 127) of every E8M0 byte; 255 is NaN."""
    s = np.asarray(scale_bytes, dtype=np.uint8).astype(np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def unpack_fp4(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] nibbles, element 2i from the low nibble of byte i."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def dequantize_mxfp4(packed, scale_bytes) -> np.ndarray:
    """W[..., n, k] = 2^(s[..., n, k // 32] - 127) * e2m1(code[..., n, k]) in float64
    (exact: a two-bit significand times a power of two)."""
    v = decode_e2m1(unpack_fp4(packed))
    sc = decode_e8m0(scale_bytes)
    if v.shape[-1] != MX_BLOCK * sc.shape[-1] or v.shape[:-1] != sc.shape[:-1]:
        raise ValueError("scale shape %s does not match codes %s" % (sc.shape, v.shape))
    return v * np.repeat(sc, MX_BLOCK, axis=-1)

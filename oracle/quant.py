"""Oracle for the 8-bit KV cache (test infrastructure only).

What the pages fix.  The xdnf.cn article (§2.3, choosing among designs, and
§6.3, combining paging with quantisation and speculative decoding) names
storing the KV cache in 8-bit integers: it cuts memory at some cost in
accuracy, and it composes with paging because quantisation changes the values
the cache holds while paging only changes how the memory is organised.
"PagedAttention 实现细节" §3.4 lists int8 among the paged backend's dtypes.

What they leave open, and the readings taken here:

* Format.  Two 8-bit code formats share one pool layout: signed int8, the
  pages' own word, and OCP FP8 E4M3 ("fn": 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals, no infinities, NaN = S.1111.111, largest
  finite value 448), the 8-bit type with native conversions on gfx950.
* Scales.  One float32 scale per pool, k_scale for keys and v_scale for values
  (per-tensor scaling: the plainest scheme; the pages give none).  Stored code
  = Q(x / scale) with the division done in float32; the cache then stands for
  decode(code) * scale.
* Rounding.  To nearest, ties to even, for both formats.
* Out of range.  E4M3: finite values beyond +-448 and +-inf saturate to +-448
  (codes 0x7E / 0xFE); NaN becomes 0x7F.  int8: saturate to [-127, 127]
  (symmetric, so Q(-y) = -Q(y)); NaN becomes 0.  Signed zeros keep their sign
  in E4M3 (0x00 / 0x80).

A second int8 form keeps one scale per (token, KV head) instead of one per
pool, the per-token form the xdnf.cn article's §2.3/§6.3 name among the
quantisation choices: each new key row and each new value row of D elements
gets s = max_d |x_d| / 127 (float32 division) and codes Q(x_d / s), so its
largest element maps to +-127.  A row of zeros has s = 0 and codes 0.  Rows
must be finite (a NaN row's codes are not specified).  The cache then stands
for decode(code) * s of that row.

The E4M3 encoder is a brute-force nearest-value search over the code table,
built from the format's definition; the int8 encoder is the nearest integer.
Pools are uint8 arrays holding the codes, with the layouts of the
16-bit pools: keys [NB, H_kv, bs, D], values [NB, H_kv, D, bs].
"""
from __future__ import annotations

import numpy as np

FORMATS = ("fp8_e4m3", "int8")
INT8_TOKEN = "int8_token"  # int8 codes with one float32 scale per (token, KV head)
E4M3_MAX = 448.0
INT8_MAX = 127


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code (float64; NaN for 0x7F and 0xFF)."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6  # subnormal: 0.mmm x 2^(1 - bias)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return sign * mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# the non-negative finite codes 0x00 .. 0x7E, in increasing order of value
_POS_VALUES = E4M3_TABLE[:0x7F]


def int8_value(code: int) -> float:
    """Value of one int8 code given as its byte (two's complement)."""
    return float(code - 256 if code >= 128 else code)


INT8_TABLE = np.array([int8_value(c) for c in range(256)], dtype=np.float64)


def decode(codes, fmt: str) -> np.ndarray:
    """Code bytes (uint8) -> float64 values."""
    table = E4M3_TABLE if fmt == "fp8_e4m3" else INT8_TABLE if fmt == "int8" else None
    if table is None:
        raise ValueError(fmt)
    return table[np.asarray(codes, dtype=np.uint8)]


def _e4m3_encode(y32: np.ndarray) -> np.ndarray:
    y = y32.astype(np.float64).ravel()
    out = np.empty(y.shape, dtype=np.uint8)
    nan = np.isnan(y)
    mag = np.where(nan, 0.0, np.abs(y))
    # nearest non-negative finite value; a tie goes to the even code
    dist = np.abs(mag[:, None] - _POS_VALUES[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    even = cand & (np.arange(0x7F)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = np.where(mag > E4M3_MAX, 0x7E, code)  # saturate (inf included)
    sign = np.signbit(y).astype(np.int64) << 7
    out[:] = np.where(nan, 0x7F, code | sign)
    return out.reshape(y32.shape)


def _int8_encode(y32: np.ndarray) -> np.ndarray:
    y = y32.astype(np.float64)
    r = np.clip(np.rint(np.where(np.isnan(y), 0.0, y)), -INT8_MAX, INT8_MAX)  # rint: ties to even
    return r.astype(np.int64).astype(np.uint8)


def encode(y32, fmt: str) -> np.ndarray:
    """float32 values -> code bytes (uint8)."""
    y32 = np.asarray(y32, dtype=np.float32)
    if fmt == "fp8_e4m3":
        return _e4m3_encode(y32)
    if fmt == "int8":
        return _int8_encode(y32)
    raise ValueError(fmt)


def to_f32(x, dtype: str) -> np.ndarray:
    """Exact float32 view of a storage array (bf16 given as uint16 bits)."""
    x = np.asarray(x)
    if dtype == "bf16":
        return (x.astype(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype in ("f32", "f16"):
        return x.astype(np.float32)
    raise ValueError(dtype)


def quantize(x, dtype: str, scale: float, fmt: str) -> np.ndarray:
    """Codes of Q(x / scale): x in storage type `dtype`, the quotient in float32."""
    q = to_f32(x, dtype) / np.float32(scale)
    return encode(q, fmt)


def dequantize(codes, scale: float, fmt: str) -> np.ndarray:
    """float64 values the codes stand for: decode(code) * scale (scale as float32)."""
    return decode(codes, fmt) * float(np.float32(scale))


def quantize_rows_int8(x, dtype: str):
    """Per-row int8: for each row (last axis) s = max |x| / 127 in float32 and codes
    Q_int8(x / s) (float32 quotient, nearest with ties to even, saturating at +-127); a
    row of zeros gets s = 0 and codes 0.  Returns (codes uint8 [..., D], scales float32 [...])."""
    x32 = to_f32(x, dtype)
    amax = np.max(np.abs(x32), axis=-1)
    scales = (amax / np.float32(INT8_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (x32 / scales[..., None]).astype(np.float32)
    codes = np.where(scales[..., None] > 0, _int8_encode(quot), np.uint8(0)).astype(np.uint8)
    return codes, scales


def dequantize_rows_int8(codes, scales) -> np.ndarray:
    """float64 values of per-row int8 codes: decode(code) * s of the row."""
    return decode(codes, "int8") * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]

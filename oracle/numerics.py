"""Number formats for the oracle, written from their definitions.

* bf16: the upper 16 bits of an IEEE binary32 (decode is exact).
* fl32: IEEE binary32 round-to-nearest-even (numpy's float32 cast).
* E4M3FN (OCP 8-bit floating point spec): 1 sign, 4 exponent bits with bias 7,
  3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448 =
  1.75 * 2^8; smallest normal 2^-6; subnormals m * 2^-9, m = 1..7.

The FP8 scaling recipe follows the pages' granularity (xyznot.com guides,
key-ideas FP8 bullet; pwwt.cn note §3): one fp32 scale per 1x128 activation
tile and per 128x128 weight block. Reading taken where the pages are silent:
scale = fl32(amax / 448) (1.0 when amax = 0); code = E4M3(fl32(x / scale)) with
round-to-nearest-even and saturation to +-448.
"""

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even) via exact binary32 steps."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, |m| in [0.5, 1)
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # 8 significant bits, RNE
    return q


def fl32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Canonical input array (bf16 bits or fp32) -> exact fp64."""
    if dtype == "bf16":
        return bf16_to_f64(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------- E4M3FN
def e4m3_encode(x32: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3FN codes (uint8), round to nearest even, saturating."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, ex = np.frexp(a)                      # a in [2^(ex-1), 2^ex)
    e = np.maximum(ex - 1, -6)               # binade; below 2^-6 the step is 2^-9
    step = np.ldexp(1.0, e - 3)
    v = np.rint(a / step) * step             # exact: a/step scales by a power of two
    v = np.minimum(v, E4M3_MAX)
    code = np.zeros(x.shape, dtype=np.uint8)
    nz = v > 0
    _, ev = np.frexp(np.where(nz, v, 1.0))
    ev = ev - 1
    sub = nz & (ev < -6)
    nor = nz & ~sub
    mant_sub = np.rint(np.where(sub, v, 0.0) / 2.0 ** -9).astype(np.int64)
    mant_nor = np.rint((np.where(nor, v, 1.0) / np.ldexp(1.0, np.where(nor, ev, 0)) - 1.0) * 8).astype(np.int64)
    exp_nor = np.where(nor, ev + 7, 0).astype(np.int64)
    c = np.where(sub, mant_sub, 0) + np.where(nor, (exp_nor << 3) | mant_nor, 0)
    code[...] = (c | np.where(neg, 0x80, 0)).astype(np.uint8)
    return code


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    val = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.ldexp(1.0, E - 7))
    val = np.where((E == 15) & (M == 7), np.nan, val)
    return sign * val


def _scale_from_amax(amax32: np.ndarray) -> np.ndarray:
    s = (amax32.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)


def quant_act_1x128(x32: np.ndarray):
    """Activations [R, C] (C % 128 == 0) -> (codes [R, C], scales [R, C/128])."""
    x = np.asarray(x32, dtype=np.float32)
    R, C = x.shape
    tiles = x.reshape(R, C // 128, 128)
    amax = np.abs(tiles).max(axis=2)
    scale = _scale_from_amax(amax)
    y = (tiles / scale[:, :, None]).astype(np.float32)          # fp32 IEEE division
    return e4m3_encode(y).reshape(R, C), scale


def quant_w_128x128(w32: np.ndarray):
    """Weights [N, K] (both % 128 == 0) -> (codes [N, K], scales [N/128, K/128])."""
    w = np.asarray(w32, dtype=np.float32)
    N, K = w.shape
    blk = w.reshape(N // 128, 128, K // 128, 128)
    amax = np.abs(blk).max(axis=(1, 3))
    scale = _scale_from_amax(amax)
    y = (blk / scale[:, None, :, None]).astype(np.float32)
    return e4m3_encode(y).reshape(N, K), scale


def dequant_act(codes, scale):
    R, C = codes.shape
    return (e4m3_decode(codes).reshape(R, C // 128, 128) * scale.astype(np.float64)[:, :, None]).reshape(R, C)


def dequant_w(codes, scale):
    N, K = codes.shape
    v = e4m3_decode(codes).reshape(N // 128, 128, K // 128, 128)
    return (v * scale.astype(np.float64)[:, None, :, None]).reshape(N, K)

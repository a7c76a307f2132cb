"""CPU oracle for appending new tokens' K/V to a paged cache.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): only tests, the smoke check and the
benchmark's CPU baseline may use it; it imports nothing from the product.

What is written ([P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 and [P3]
"内存优化：KV Cache管理、PagedAttention原理与内存池配置", paged-pool section: the cache of a
request grows block by block, and a block table maps its logical blocks to physical ones;
[P2] vLLM architecture deep-dive §2.1: the decode mode produces one new token per step):
new token t of sequence s at logical position p is stored in physical block
block_tables[s][p // block_size], slot p % block_size, for every KV head, its K and V rows
rounded to the pool's storage type.

Storage rounding (the pages name only "FP8" for the quantised cache, [P2] §4.2):
  * f32 pools keep the value; f16 and bf16 pools round to nearest, ties to even.
  * fp8-e4m3 (OCP: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
    infinities, S.1111.111 = NaN, largest finite 448): y = x / scale, both fp32 and the
    division rounded to fp32 as IEEE division does; then y is rounded to the nearest
    e4m3 value, ties to an even mantissa; magnitudes beyond 448 (infinities included)
    saturate to +-448, and NaN becomes the code 0x7F.
"""
from __future__ import annotations

import math

import numpy as np

FP8_MAX = 448.0


def _fp8_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3_encode_scalar(y: float) -> int:
    """One fp32 value (already divided by the scale) -> e4m3 code, from the definition."""
    if math.isnan(y):
        return 0x7F
    sign = 0x80 if (y < 0 or (y == 0 and math.copysign(1.0, y) < 0)) else 0x00
    a = abs(y)
    if a >= FP8_MAX:
        return sign | 0x7E  # saturate (448 = 1.75 * 2^8)
    if a < 2.0 ** -6:
        # subnormal range: multiples of 2^-9, round half to even
        q = a / 2.0 ** -9
        m = math.floor(q)
        r = q - m
        if r > 0.5 or (r == 0.5 and m % 2 == 1):
            m += 1
        if m == 8:  # rounded up to the smallest normal 2^-6 = exponent field 1
            return sign | (1 << 3)
        return sign | m
    e = math.floor(math.log2(a))
    # guard against log2 rounding at exact powers of two
    if 2.0 ** e > a:
        e -= 1
    if 2.0 ** (e + 1) <= a:
        e += 1
    step = 2.0 ** (e - 3)  # spacing of the 3-bit mantissa in [2^e, 2^(e+1))
    q = a / step           # in [8, 16)
    n = math.floor(q)
    r = q - n
    if r > 0.5 or (r == 0.5 and n % 2 == 1):
        n += 1
    if n == 16:
        n = 8
        e += 1
    if e > 8 or (e == 8 and n > 14):
        return sign | 0x7E  # rounded beyond 448: saturate
    return sign | ((e + 7) << 3) | (n - 8)


def fp8_e4m3_encode(y: np.ndarray) -> np.ndarray:
    y = np.asarray(y, dtype=np.float32)
    flat = [fp8_e4m3_encode_scalar(float(v)) for v in y.reshape(-1)]
    return np.asarray(flat, dtype=np.uint8).reshape(y.shape)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bits, round to nearest, ties to even (NaN stays NaN)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return r


def decode_src(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored new-token values -> float32 (exact)."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        u = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32)
    raise ValueError(dtype)


def encode(x_f32: np.ndarray, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """float32 values -> pool storage (see the module text for each type)."""
    x = np.asarray(x_f32, dtype=np.float32)
    if kv_dtype == "f32":
        return x.copy()
    if kv_dtype == "f16":
        return x.astype(np.float16)
    if kv_dtype == "bf16":
        return bf16_encode(x)
    if kv_dtype == "fp8_e4m3":
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            y = x / np.float32(scale)
        return fp8_e4m3_encode(y)
    raise ValueError(kv_dtype)


def append_kv(k_pool, v_pool, block_tables, seq_ids, positions, k_new, v_new, src_dtype: str,
              kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0):
    """Copies of the pools with each new token's K and V rows written into its slot.

    k_pool / v_pool: [num_blocks][num_kv_heads][block_size][head_dim] storage arrays.
    k_new / v_new:   [T][num_kv_heads][head_dim] in src_dtype storage.
    Token t belongs to sequence seq_ids[t] at logical position positions[t].
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    nb, hkv, bs, d = kp.shape
    for t in range(len(seq_ids)):
        s = int(seq_ids[t])
        p = int(positions[t])
        b = int(block_tables[s][p // bs])
        if not (0 <= b < nb):
            raise IndexError(f"block {b} for sequence {s} position {p} outside the pool")
        slot = p % bs
        kp[b, :, slot, :] = encode(decode_src(k_new[t], src_dtype), kv_dtype, k_scale)
        vp[b, :, slot, :] = encode(decode_src(v_new[t], src_dtype), kv_dtype, v_scale)
    return kp, vp

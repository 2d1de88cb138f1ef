"""Bit-level readers and writers of the four block formats, in plain numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source of each layout:

* Q8_0, Q4_K, Q6_K -- VTE (kyuubyn.github.io/VTE), feature list: these three
  GGUF block types are dequantized byte for byte in llama.cpp's reference
  layout.  The pages name the layout but do not print it; the byte maps below
  are GGUF's published block definitions as this library reads them (see the
  layout table in each function).  hipEngine 0.3.0, "GGUF Support", lists the
  same three types (plus Q5_K) as the tensor payload of a Q4_K_M file.
* Q5_K -- hipEngine 0.3.0, "GGUF Support": 31% of the Q4_K_M tensor payload
  (the MoE expert-down projections).  The page names the type only; the byte
  map below is GGUF's published Q5_K block as this library reads it.
* INT4_G128 -- "Costruire un runtime di inference LLM da zero" (datastack.it),
  "Tre bug che insegnano": symmetric INT4, one scale per 128 weights.  The
  page gives no byte layout; this library's reading is a codes plane followed
  by a scales plane (below).

All fp16 fields are IEEE binary16, little-endian.  Tensors are row-major: a row
of ``cols`` weights is ``cols / QK`` consecutive blocks and rows follow each
other with no padding.

Field arrays ("fields") used by ``pack``/``unpack``:

  q8_0      d_bits u16[rows, nb], q i8[rows, cols]
  q4_k      d_bits u16[rows, nb], dmin_bits u16[rows, nb],
            sc u8[rows, nb, 8] (0..63), m u8[rows, nb, 8] (0..63),
            u u8[rows, cols] (0..15)
  q5_k      d_bits, dmin_bits, sc, m as q4_k; u u8[rows, cols] (0..31)
  q6_k      d_bits u16[rows, nb], sc i8[rows, nb, 16], q u8[rows, cols] (0..63)
  int4_g128 s_bits u16[rows, cols/128], q i8[rows, cols] (-8..7)

Codes are indexed by the weight's column, so ``q[r, k]`` is the code of W[r, k].
"""
from __future__ import annotations

import numpy as np

from .fp import fp16_bits_to_f64

FORMATS = ("q8_0", "q4_k", "q6_k", "int4_g128", "q5_k")
QK = {"q8_0": 32, "q4_k": 256, "q6_k": 256, "int4_g128": 128, "q5_k": 256}
BLOCK_BYTES = {"q8_0": 34, "q4_k": 144, "q6_k": 210, "q5_k": 176}


def _check_shape(fmt: str, rows: int, cols: int) -> None:
    if fmt not in QK:
        raise ValueError(f"unknown format {fmt!r}")
    if rows < 1 or cols < 1 or cols % QK[fmt]:
        raise ValueError(f"{fmt}: bad shape {rows}x{cols} (cols must be a multiple of {QK[fmt]})")


def packed_size(fmt: str, rows: int, cols: int) -> int:
    _check_shape(fmt, rows, cols)
    if fmt == "int4_g128":
        return rows * cols // 2 + rows * (cols // 128) * 2
    return rows * (cols // QK[fmt]) * BLOCK_BYTES[fmt]


def _le16(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    return lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)


def _put_le16(dst: np.ndarray, bits: np.ndarray) -> None:
    bits = np.asarray(bits, dtype=np.uint16)
    dst[..., 0] = bits & 0xFF
    dst[..., 1] = bits >> 8


# ----------------------------------------------------------------------------
# Q8_0: 32 weights, 34 bytes.
#   bytes [0, 2)   d, fp16
#   bytes [2, 34)  q[0..31], int8, q[i] is the code of weight i
#   w_i = d * q_i
# ----------------------------------------------------------------------------
def _pack_q8_0(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 32
    blk = np.zeros((rows, nb, 34), np.uint8)
    _put_le16(blk[:, :, 0:2], f["d_bits"])
    blk[:, :, 2:34] = np.asarray(f["q"], np.int8).reshape(rows, nb, 32).view(np.uint8)
    return blk.reshape(-1)


def _unpack_q8_0(data: np.ndarray, rows: int, cols: int) -> dict:
    nb = cols // 32
    blk = data.reshape(rows, nb, 34)
    d_bits = _le16(blk[:, :, 0], blk[:, :, 1])
    q = np.ascontiguousarray(blk[:, :, 2:34]).view(np.int8).reshape(rows, cols)
    return {"d_bits": d_bits, "q": q}


def _dequant_q8_0(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 32
    d = fp16_bits_to_f64(f["d_bits"])                         # [rows, nb]
    q = f["q"].astype(np.float64).reshape(rows, nb, 32)
    return (d[:, :, None] * q).reshape(rows, cols)


# ----------------------------------------------------------------------------
# Q4_K: 256 weights, 144 bytes, eight sub-blocks of 32.
#   bytes [0, 2)    d, fp16       (scale of the sub-block scales)
#   bytes [2, 4)    dmin, fp16    (scale of the sub-block mins)
#   bytes [4, 16)   scales[12]: eight 6-bit scales sc_j and eight 6-bit mins m_j
#        j < 4:  sc_j = scales[j] & 63            m_j = scales[j+4] & 63
#        j >= 4: sc_j = (scales[j+4] & 15) | (scales[j-4] >> 6) << 4
#                m_j  = (scales[j+4] >> 4) | (scales[j]   >> 6) << 4
#   bytes [16, 144) qs[128]: weight t = 64c + 32h + l (c < 4, h < 2, l < 32)
#        has code u = (qs[32c + l] >> 4h) & 15 and sub-block s = 2c + h = t // 32
#   w_t = d * sc_s * u - dmin * m_s
# ----------------------------------------------------------------------------
def q4_k_scales_to_bytes(sc: np.ndarray, m: np.ndarray) -> np.ndarray:
    sc = np.asarray(sc, np.uint8)
    m = np.asarray(m, np.uint8)
    out = np.zeros(sc.shape[:-1] + (12,), np.uint8)
    for j in range(4):
        out[..., j] = (sc[..., j] & 63) | ((sc[..., j + 4] >> 4) << 6)
        out[..., j + 4] = (m[..., j] & 63) | ((m[..., j + 4] >> 4) << 6)
        out[..., j + 8] = (sc[..., j + 4] & 15) | ((m[..., j + 4] & 15) << 4)
    return out


def q4_k_bytes_to_scales(scales: np.ndarray):
    s = np.asarray(scales, np.uint8)
    sc = np.zeros(s.shape[:-1] + (8,), np.uint8)
    m = np.zeros(s.shape[:-1] + (8,), np.uint8)
    for j in range(8):
        if j < 4:
            sc[..., j] = s[..., j] & 63
            m[..., j] = s[..., j + 4] & 63
        else:
            sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
            m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, m


def q4_k_codes_to_qs(u: np.ndarray) -> np.ndarray:
    """u[..., 256] (0..15) -> qs[..., 128]."""
    u = np.asarray(u, np.uint8).reshape(u.shape[:-1] + (4, 2, 32))   # [c, h, l]
    qs = u[..., 0, :] | (u[..., 1, :] << 4)                          # [c, l]
    return qs.reshape(qs.shape[:-2] + (128,))


def q4_k_qs_to_codes(qs: np.ndarray) -> np.ndarray:
    """qs[..., 128] -> u[..., 256] with weight t = 64c + 32h + l."""
    q = np.asarray(qs, np.uint8).reshape(qs.shape[:-1] + (4, 32))    # [c, l]
    u = np.stack([q & 15, q >> 4], axis=-2)                           # [c, h, l]
    return u.reshape(qs.shape[:-1] + (256,))


def _pack_q4_k(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 256
    blk = np.zeros((rows, nb, 144), np.uint8)
    _put_le16(blk[:, :, 0:2], f["d_bits"])
    _put_le16(blk[:, :, 2:4], f["dmin_bits"])
    blk[:, :, 4:16] = q4_k_scales_to_bytes(f["sc"], f["m"])
    blk[:, :, 16:144] = q4_k_codes_to_qs(np.asarray(f["u"]).reshape(rows, nb, 256))
    return blk.reshape(-1)


def _unpack_q4_k(data: np.ndarray, rows: int, cols: int) -> dict:
    nb = cols // 256
    blk = data.reshape(rows, nb, 144)
    sc, m = q4_k_bytes_to_scales(blk[:, :, 4:16])
    return {"d_bits": _le16(blk[:, :, 0], blk[:, :, 1]),
            "dmin_bits": _le16(blk[:, :, 2], blk[:, :, 3]),
            "sc": sc, "m": m,
            "u": q4_k_qs_to_codes(blk[:, :, 16:144]).reshape(rows, cols)}


def _dequant_q4_k(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 256
    d = fp16_bits_to_f64(f["d_bits"])[:, :, None, None]               # [r, b, 1, 1]
    dmin = fp16_bits_to_f64(f["dmin_bits"])[:, :, None, None]
    sc = f["sc"].astype(np.float64)[:, :, :, None]                    # [r, b, s, 1]
    m = f["m"].astype(np.float64)[:, :, :, None]
    u = f["u"].astype(np.float64).reshape(rows, nb, 8, 32)            # [r, b, s, l]
    a = d * sc * u          # exact: at most 11 + 6 + 4 significant bits
    b = dmin * m            # exact: at most 11 + 6 significant bits
    w = a - b
    # TwoSum error of a + (-b): zero means w is the exact difference.
    bb = w - a
    err = (a - (w - bb)) + (-b - bb)
    if np.any(err != 0):
        raise AssertionError("Q4_K weight not exact in float64")
    return w.reshape(rows, cols)


# ----------------------------------------------------------------------------
# Q6_K: 256 weights, 210 bytes, sixteen sub-blocks of 16.
#   bytes [0, 128)    ql[128]: low 4 bits of the 6-bit codes
#   bytes [128, 192)  qh[64]:  high 2 bits of the 6-bit codes
#   bytes [192, 208)  sc[16]:  int8 sub-block scales
#   bytes [208, 210)  d, fp16
#   weight t = 128h + 32g + l (h < 2, g < 4, l < 32):
#        low  = (ql[64h + 32(g & 1) + l] >> 4(g >> 1)) & 15
#        high = (qh[32h + l] >> 2g) & 3
#        q6 = low | high << 4,   sub-block = 8h + 2g + (l >> 4) = t // 16
#   w_t = d * sc[t // 16] * (q6 - 32)
# ----------------------------------------------------------------------------
def q6_k_codes_to_bytes(q: np.ndarray):
    """q[..., 256] (0..63) -> (ql[..., 128], qh[..., 64])."""
    q = np.asarray(q, np.uint8).reshape(q.shape[:-1] + (2, 4, 32))   # [h, g, l]
    lo = q & 15
    hi = q >> 4
    ql = np.concatenate([lo[..., 0, :] | (lo[..., 2, :] << 4),       # ql[64h + l]
                         lo[..., 1, :] | (lo[..., 3, :] << 4)],      # ql[64h + 32 + l]
                        axis=-1)                                      # [h, 64]
    qh = hi[..., 0, :] | (hi[..., 1, :] << 2) | (hi[..., 2, :] << 4) | (hi[..., 3, :] << 6)
    return (ql.reshape(ql.shape[:-2] + (128,)), qh.reshape(qh.shape[:-2] + (64,)))


def q6_k_bytes_to_codes(ql: np.ndarray, qh: np.ndarray) -> np.ndarray:
    ql = np.asarray(ql, np.uint8).reshape(ql.shape[:-1] + (2, 2, 32))   # [h, half, l]
    qh = np.asarray(qh, np.uint8).reshape(qh.shape[:-1] + (2, 32))      # [h, l]
    out = np.zeros(ql.shape[:-3] + (2, 4, 32), np.uint8)                # [h, g, l]
    for g in range(4):
        low = (ql[..., :, g & 1, :] >> (4 * (g >> 1))) & 15
        high = (qh >> (2 * g)) & 3
        out[..., :, g, :] = low | (high << 4)
    return out.reshape(out.shape[:-3] + (256,))


def _pack_q6_k(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 256
    blk = np.zeros((rows, nb, 210), np.uint8)
    ql, qh = q6_k_codes_to_bytes(np.asarray(f["q"]).reshape(rows, nb, 256))
    blk[:, :, 0:128] = ql
    blk[:, :, 128:192] = qh
    blk[:, :, 192:208] = np.asarray(f["sc"], np.int8).view(np.uint8)
    _put_le16(blk[:, :, 208:210], f["d_bits"])
    return blk.reshape(-1)


def _unpack_q6_k(data: np.ndarray, rows: int, cols: int) -> dict:
    nb = cols // 256
    blk = data.reshape(rows, nb, 210)
    q = q6_k_bytes_to_codes(blk[:, :, 0:128], blk[:, :, 128:192]).reshape(rows, cols)
    sc = np.ascontiguousarray(blk[:, :, 192:208]).view(np.int8)
    return {"d_bits": _le16(blk[:, :, 208], blk[:, :, 209]), "sc": sc, "q": q}


def _dequant_q6_k(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 256
    d = fp16_bits_to_f64(f["d_bits"])[:, :, None, None]               # [r, b, 1, 1]
    sc = f["sc"].astype(np.float64)[:, :, :, None]                    # [r, b, 16, 1]
    q = f["q"].astype(np.float64).reshape(rows, nb, 16, 16) - 32.0    # [r, b, sub, i]
    return (d * sc * q).reshape(rows, cols)


# ----------------------------------------------------------------------------
# INT4_G128: symmetric 4-bit, one fp16 scale per 128 consecutive weights of a row.
#   codes plane, bytes [0, rows*cols/2): row r occupies cols/2 bytes; byte j of
#        the row holds u_{2j} in bits 0-3 and u_{2j+1} in bits 4-7, u = q + 8
#   scales plane, bytes [rows*cols/2, +rows*(cols/128)*2): fp16 s[r][g]
#   w_k = s_{k // 128} * (u_k - 8)
# ----------------------------------------------------------------------------
def _pack_int4_g128(f: dict, rows: int, cols: int) -> np.ndarray:
    q = np.asarray(f["q"], np.int8).reshape(rows, cols // 2, 2)
    u = (q.astype(np.int16) + 8).astype(np.uint8)
    codes = (u[:, :, 0] | (u[:, :, 1] << 4)).reshape(-1)
    s = np.zeros((rows, cols // 128, 2), np.uint8)
    _put_le16(s, f["s_bits"])
    return np.concatenate([codes, s.reshape(-1)])


def _unpack_int4_g128(data: np.ndarray, rows: int, cols: int) -> dict:
    ncode = rows * cols // 2
    codes = data[:ncode].reshape(rows, cols // 2)
    u = np.stack([codes & 15, codes >> 4], axis=-1).reshape(rows, cols)
    s = data[ncode:].reshape(rows, cols // 128, 2)
    return {"s_bits": _le16(s[:, :, 0], s[:, :, 1]),
            "q": (u.astype(np.int16) - 8).astype(np.int8)}


def _dequant_int4_g128(f: dict, rows: int, cols: int) -> np.ndarray:
    s = fp16_bits_to_f64(f["s_bits"])[:, :, None]                     # [r, g, 1]
    q = f["q"].astype(np.float64).reshape(rows, cols // 128, 128)
    return (s * q).reshape(rows, cols)


# ----------------------------------------------------------------------------
# Q5_K: 256 weights, 176 bytes, eight sub-blocks of 32.
#   bytes [0, 2)    d, fp16;  bytes [2, 4) dmin, fp16
#   bytes [4, 16)   scales[12]: the six-bit scales and mins, packed as in Q4_K
#   bytes [16, 48)  qh[32]: bit 2c + h of qh[l] is the fifth code bit of weight
#                   t = 64c + 32h + l
#   bytes [48, 176) qs[128]: the low four code bits, arranged as Q4_K's qs
#        (weight t = 64c + 32h + l takes nibble h of qs[32c + l])
#   u = low | high << 4 (0..31),  sub-block s = 2c + h = t // 32
#   w_t = d * sc_s * u - dmin * m_s
# ----------------------------------------------------------------------------
def q5_k_codes_to_bytes(u: np.ndarray):
    """u[..., 256] (0..31) -> (qh[..., 32], qs[..., 128])."""
    u = np.asarray(u, np.uint8)
    qs = q4_k_codes_to_qs(u & 15)
    hi = (u >> 4).reshape(u.shape[:-1] + (8, 32))                     # [s = 2c + h, l]
    qh = np.zeros(u.shape[:-1] + (32,), np.uint8)
    for s in range(8):
        qh |= (hi[..., s, :] << s).astype(np.uint8)
    return qh, qs


def q5_k_bytes_to_codes(qh: np.ndarray, qs: np.ndarray) -> np.ndarray:
    """(qh[..., 32], qs[..., 128]) -> u[..., 256] with weight t = 64c + 32h + l."""
    low = q4_k_qs_to_codes(qs).reshape(qs.shape[:-1] + (8, 32))     # [s, l]
    qh = np.asarray(qh, np.uint8)
    high = np.stack([(qh >> s) & 1 for s in range(8)], axis=-2)      # [s, l]
    return (low | (high << 4)).reshape(qs.shape[:-1] + (256,))


def _pack_q5_k(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 256
    blk = np.zeros((rows, nb, 176), np.uint8)
    _put_le16(blk[:, :, 0:2], f["d_bits"])
    _put_le16(blk[:, :, 2:4], f["dmin_bits"])
    blk[:, :, 4:16] = q4_k_scales_to_bytes(f["sc"], f["m"])
    qh, qs = q5_k_codes_to_bytes(np.asarray(f["u"]).reshape(rows, nb, 256))
    blk[:, :, 16:48] = qh
    blk[:, :, 48:176] = qs
    return blk.reshape(-1)


def _unpack_q5_k(data: np.ndarray, rows: int, cols: int) -> dict:
    nb = cols // 256
    blk = data.reshape(rows, nb, 176)
    sc, m = q4_k_bytes_to_scales(blk[:, :, 4:16])
    return {"d_bits": _le16(blk[:, :, 0], blk[:, :, 1]),
            "dmin_bits": _le16(blk[:, :, 2], blk[:, :, 3]),
            "sc": sc, "m": m,
            "u": q5_k_bytes_to_codes(blk[:, :, 16:48], blk[:, :, 48:176]).reshape(rows, cols)}


def _dequant_q5_k(f: dict, rows: int, cols: int) -> np.ndarray:
    nb = cols // 256
    d = fp16_bits_to_f64(f["d_bits"])[:, :, None, None]               # [r, b, 1, 1]
    dmin = fp16_bits_to_f64(f["dmin_bits"])[:, :, None, None]
    sc = f["sc"].astype(np.float64)[:, :, :, None]                    # [r, b, s, 1]
    m = f["m"].astype(np.float64)[:, :, :, None]
    u = f["u"].astype(np.float64).reshape(rows, nb, 8, 32)            # [r, b, s, l]
    a = d * sc * u          # exact: at most 11 + 6 + 5 significant bits
    b = dmin * m            # exact: at most 11 + 6 significant bits
    w = a - b
    bb = w - a              # TwoSum error term of a + (-b) must vanish
    err = (a - (w - bb)) + (-b - bb)
    if np.any(err != 0):
        raise AssertionError("Q5_K weight not exact in float64")
    return w.reshape(rows, cols)


_PACK = {"q8_0": _pack_q8_0, "q4_k": _pack_q4_k, "q6_k": _pack_q6_k,
         "int4_g128": _pack_int4_g128, "q5_k": _pack_q5_k}
_UNPACK = {"q8_0": _unpack_q8_0, "q4_k": _unpack_q4_k, "q6_k": _unpack_q6_k,
           "int4_g128": _unpack_int4_g128, "q5_k": _unpack_q5_k}
_DEQUANT = {"q8_0": _dequant_q8_0, "q4_k": _dequant_q4_k, "q6_k": _dequant_q6_k,
            "int4_g128": _dequant_int4_g128, "q5_k": _dequant_q5_k}

_RANGES = {  # field -> (lo, hi) inclusive, for range validation of codes
    "q8_0": {"q": (-128, 127)},
    "q4_k": {"sc": (0, 63), "m": (0, 63), "u": (0, 15)},
    "q5_k": {"sc": (0, 63), "m": (0, 63), "u": (0, 31)},
    "q6_k": {"sc": (-128, 127), "q": (0, 63)},
    "int4_g128": {"q": (-8, 7)},
}


def pack(fmt: str, fields: dict, rows: int, cols: int) -> np.ndarray:
    """Fields -> canonical packed bytes (uint8, length packed_size)."""
    _check_shape(fmt, rows, cols)
    for name, (lo, hi) in _RANGES[fmt].items():
        v = np.asarray(fields[name])
        if v.size and (v.min() < lo or v.max() > hi):
            raise ValueError(f"{fmt}.{name} out of range [{lo}, {hi}]")
    out = _PACK[fmt](fields, rows, cols)
    assert out.dtype == np.uint8 and out.size == packed_size(fmt, rows, cols)
    return out


def unpack(fmt: str, data, rows: int, cols: int) -> dict:
    _check_shape(fmt, rows, cols)
    data = np.asarray(data, np.uint8).reshape(-1)
    if data.size != packed_size(fmt, rows, cols):
        raise ValueError("packed size mismatch")
    return _UNPACK[fmt](data, rows, cols)


def dequant64(fmt: str, data, rows: int, cols: int) -> np.ndarray:
    """Exact value of every weight, float64 [rows, cols]."""
    return _DEQUANT[fmt](unpack(fmt, data, rows, cols), rows, cols)


def dequant32(fmt: str, data, rows: int, cols: int) -> np.ndarray:
    """float32 dequantization: the exact value rounded once to nearest-even.

    Q8_0, Q6_K and INT4 products fit in binary32's 24-bit significand, so the
    float32 value equals the exact one; Q4_K and Q5_K round once, at the
    subtraction.
    """
    return dequant64(fmt, data, rows, cols).astype(np.float32)


def row_slice(fmt: str, data, rows: int, cols: int, r0: int, r1: int) -> np.ndarray:
    """Packed bytes of rows [r0, r1) as a standalone (r1 - r0) x cols tensor."""
    _check_shape(fmt, rows, cols)
    data = np.asarray(data, np.uint8).reshape(-1)
    if not 0 <= r0 < r1 <= rows:
        raise ValueError("bad row range")
    if fmt == "int4_g128":
        cb, sb = cols // 2, (cols // 128) * 2
        codes = data[r0 * cb:r1 * cb]
        base = rows * cb
        scales = data[base + r0 * sb:base + r1 * sb]
        return np.concatenate([codes, scales])
    rb = (cols // QK[fmt]) * BLOCK_BYTES[fmt]
    return data[r0 * rb:r1 * rb].copy()

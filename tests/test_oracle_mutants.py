"""Planted mistakes in the oracle (on the CPU) must each be caught by some pin.

Every mutant below is a plausible slip in a block decoder or in the GEMV: a
swapped nibble, a wrong shift or index, a dropped or sign-flipped term, a wrong
byte order, a transposed operand.  The test patches the mutant into the oracle,
runs the whole pin suite, and requires at least one pin to fail.
"""
import numpy as np
import pytest

import oracle
import oracle.formats as F
import oracle.fp as FP
import oracle.gemv as G
from oracle_pins import failing_pins


def _q4k_codes_swapped(qs):
    q = np.asarray(qs, np.uint8).reshape(qs.shape[:-1] + (4, 32))
    u = np.stack([q >> 4, q & 15], axis=-2)
    return u.reshape(qs.shape[:-1] + (256,))


def _q4k_scales_wrong_index(scales):
    sc, m = Q4K_SCALES_ORIG(scales)
    s = np.asarray(scales, np.uint8)
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j] >> 6) << 4)   # j instead of j-4
    return sc, m


def _q4k_dequant(sign):
    def f(fields, rows, cols):
        nb = cols // 256
        d = FP.fp16_bits_to_f64(fields["d_bits"])[:, :, None, None]
        dmin = FP.fp16_bits_to_f64(fields["dmin_bits"])[:, :, None, None]
        sc = fields["sc"].astype(np.float64)[:, :, :, None]
        m = fields["m"].astype(np.float64)[:, :, :, None]
        u = fields["u"].astype(np.float64).reshape(rows, nb, 8, 32)
        return (d * sc * u + sign * dmin * m).reshape(rows, cols)
    return f


def _q6k_codes_wrong_qh_shift(ql, qh):
    ql = np.asarray(ql, np.uint8).reshape(ql.shape[:-1] + (2, 2, 32))
    qh = np.asarray(qh, np.uint8).reshape(qh.shape[:-1] + (2, 32))
    out = np.zeros(ql.shape[:-3] + (2, 4, 32), np.uint8)
    for g in range(4):
        out[..., :, g, :] = ((ql[..., :, g & 1, :] >> (4 * (g >> 1))) & 15) | (((qh >> g) & 3) << 4)
    return out.reshape(out.shape[:-3] + (256,))


def _q6k_codes_halves_swapped(ql, qh):
    ql = np.asarray(ql, np.uint8).reshape(ql.shape[:-1] + (2, 2, 32))
    qh = np.asarray(qh, np.uint8).reshape(qh.shape[:-1] + (2, 32))
    out = np.zeros(ql.shape[:-3] + (2, 4, 32), np.uint8)
    for g in range(4):
        out[..., :, g, :] = ((ql[..., :, g >> 1, :] >> (4 * (g & 1))) & 15) | (((qh >> (2 * g)) & 3) << 4)
    return out.reshape(out.shape[:-3] + (256,))


def _q6k_dequant(offset, group):
    def f(fields, rows, cols):
        nb = cols // 256
        d = FP.fp16_bits_to_f64(fields["d_bits"])[:, :, None, None]
        sc = fields["sc"].astype(np.float64)
        q = fields["q"].astype(np.float64).reshape(rows, nb, 256 // group, group) - offset
        if group == 16:
            s = sc[:, :, :, None]
        else:  # sub-blocks of 32 reading every other scale
            s = sc[:, :, ::2, None]
        return (d * s * q).reshape(rows, cols)
    return f


def _q5k_codes(bit_of, high_weight):
    def f(qh, qs):
        low = F.q4_k_qs_to_codes(qs).reshape(qs.shape[:-1] + (8, 32))
        qh = np.asarray(qh, np.uint8)
        high = np.stack([(qh >> bit_of(s)) & 1 for s in range(8)], axis=-2)
        return (low + high * high_weight).astype(np.uint8).reshape(qs.shape[:-1] + (256,))
    return f


def _q5k_unpack_planes_swapped(data, rows, cols):
    nb = cols // 256
    blk = data.reshape(rows, nb, 176)
    sc, m = F.q4_k_bytes_to_scales(blk[:, :, 4:16])
    return {"d_bits": blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8),
            "dmin_bits": blk[:, :, 2].astype(np.uint16) | (blk[:, :, 3].astype(np.uint16) << 8),
            "sc": sc, "m": m,
            "u": F.q5_k_bytes_to_codes(blk[:, :, 144:176], blk[:, :, 16:144]).reshape(rows, cols)}


def _q8_unpack_big_endian(data, rows, cols):
    nb = cols // 32
    blk = data.reshape(rows, nb, 34)
    return {"d_bits": (blk[:, :, 0].astype(np.uint16) << 8) | blk[:, :, 1],
            "q": np.ascontiguousarray(blk[:, :, 2:34]).view(np.int8).reshape(rows, cols)}


def _int4_unpack(swap, offset):
    def f(data, rows, cols):
        ncode = rows * cols // 2
        codes = data[:ncode].reshape(rows, cols // 2)
        pair = [codes >> 4, codes & 15] if swap else [codes & 15, codes >> 4]
        u = np.stack(pair, axis=-1).reshape(rows, cols)
        s = data[ncode:].reshape(rows, cols // 128, 2)
        return {"s_bits": s[:, :, 0].astype(np.uint16) | (s[:, :, 1].astype(np.uint16) << 8),
                "q": (u.astype(np.int16) - offset).astype(np.int8)}
    return f


def _fp16_bias16(bits):
    return FP_ORIG(bits) / 2.0


def _gemv_transposed(fmt, data, rows, cols, x, x_dtype, row_chunk=4096):
    x64 = G.x_to_f64(x, x_dtype).reshape(-1, cols)
    w = F.dequant64(fmt, data, rows, cols)
    return x64 @ w.reshape(cols, rows)


def _gemv_drop_last_col(fmt, data, rows, cols, x, x_dtype, row_chunk=4096):
    x64 = G.x_to_f64(x, x_dtype).reshape(-1, cols)
    w = F.dequant64(fmt, data, rows, cols)
    return x64[:, :-1] @ w[:, :-1].T


def _normwise(axis, reduce, zero_guard_one):
    def f(y, y64):
        y = np.asarray(y, np.float64).reshape(np.shape(y64))
        y64 = np.asarray(y64, np.float64)
        num = reduce(np.abs(y - y64), axis=axis)
        den = np.max(np.abs(y64), axis=axis)
        if zero_guard_one:       # the earlier guard: an all-zero row divided by 1
            return num / np.where(den == 0, 1.0, den)
        return np.where(den == 0, np.where(num == 0, 0.0, np.inf), num / np.where(den == 0, 1.0, den))
    return f


def _x_to_f64_swapped(x, x_dtype):
    x = np.asarray(x)
    if x_dtype == "f16":
        return FP.bf16_bits_to_f64(x.view(np.uint16))
    if x_dtype == "bf16":
        return FP.fp16_bits_to_f64(x)
    return X_ORIG(x, x_dtype)


def _bound_signed(fmt, data, rows, cols, x, x_dtype, row_chunk=4096):
    x64 = np.abs(G.x_to_f64(x, x_dtype).reshape(-1, cols))
    return G.gamma(cols + 1) * (x64 @ F.dequant64(fmt, data, rows, cols).T)


def _bound_gamma_k(fmt, data, rows, cols, x, x_dtype, row_chunk=4096):
    return BOUND_ORIG(fmt, data, rows, cols, x, x_dtype) * (G.gamma(cols) / G.gamma(cols + 1))


def _swiglu_swapped(fmt, gate_data, up_data, rows, cols, x, x_dtype, row_ids=None):
    return SWIGLU_ORIG(fmt, up_data, gate_data, rows, cols, x, x_dtype, row_ids)


def _silu_sigmoid(g):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


X_ORIG = G.x_to_f64
BOUND_ORIG = G.elementwise_bound
FP_ORIG = FP.fp16_bits_to_f64
Q4K_SCALES_ORIG = F.q4_k_bytes_to_scales
SWIGLU_ORIG = G.swiglu64

MUTANTS = {
    "q4_k nibbles swapped": [(F, "q4_k_qs_to_codes", _q4k_codes_swapped)],
    "q4_k scale high bits from wrong byte": [(F, "q4_k_bytes_to_scales", _q4k_scales_wrong_index)],
    "q4_k min term dropped": [(F._DEQUANT, "q4_k", _q4k_dequant(0.0))],
    "q4_k min added": [(F._DEQUANT, "q4_k", _q4k_dequant(+1.0))],
    "q6_k qh shift g not 2g": [(F, "q6_k_bytes_to_codes", _q6k_codes_wrong_qh_shift)],
    "q6_k ql halves swapped": [(F, "q6_k_bytes_to_codes", _q6k_codes_halves_swapped)],
    "q6_k offset 31": [(F._DEQUANT, "q6_k", _q6k_dequant(31.0, 16))],
    "q6_k sub-blocks of 32": [(F._DEQUANT, "q6_k", _q6k_dequant(32.0, 32))],
    "q5_k fifth bit at 4h + c": [(F, "q5_k_bytes_to_codes", _q5k_codes(lambda s: 4 * (s & 1) + (s >> 1), 16))],
    "q5_k fifth bit worth 32": [(F, "q5_k_bytes_to_codes", _q5k_codes(lambda s: s, 32))],
    "q5_k qs before qh": [(F._UNPACK, "q5_k", _q5k_unpack_planes_swapped)],
    "q5_k min term dropped": [(F._DEQUANT, "q5_k", _q4k_dequant(0.0))],
    "q8_0 d big-endian": [(F._UNPACK, "q8_0", _q8_unpack_big_endian)],
    "int4 nibbles swapped": [(F._UNPACK, "int4_g128", _int4_unpack(True, 8))],
    "int4 offset 7": [(F._UNPACK, "int4_g128", _int4_unpack(False, 7))],
    "fp16 exponent bias 16": [(F, "fp16_bits_to_f64", _fp16_bias16)],
    "gemv transposed operand": [(G, "gemv64", _gemv_transposed), (oracle, "gemv64", _gemv_transposed)],
    "gemv drops last column": [(G, "gemv64", _gemv_drop_last_col), (oracle, "gemv64", _gemv_drop_last_col)],
    "gate over the batch axis": [(oracle, "normwise_rel_err", _normwise(0, np.max, False))],
    "gate mean in place of max": [(oracle, "normwise_rel_err", _normwise(-1, np.mean, False))],
    "gate divides an all-zero row by one": [(oracle, "normwise_rel_err", _normwise(-1, np.max, True))],
    "activations f16 and bf16 swapped": [(G, "x_to_f64", _x_to_f64_swapped), (oracle, "x_to_f64", _x_to_f64_swapped)],
    "bound without |W|": [(oracle, "elementwise_bound", _bound_signed)],
    "bound gamma_K": [(oracle, "elementwise_bound", _bound_gamma_k)],
    "swiglu gate and up swapped": [(G, "swiglu64", _swiglu_swapped), (oracle, "swiglu64", _swiglu_swapped)],
    "swiglu sigmoid in place of silu": [(G, "silu64", _silu_sigmoid), (oracle, "silu64", _silu_sigmoid)],
}


def test_unmutated_oracle_passes_every_pin():
    assert failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for target, attr, repl in MUTANTS[name]:
        if isinstance(target, dict):
            monkeypatch.setitem(target, attr, repl)
        else:
            monkeypatch.setattr(target, attr, repl)
    caught = failing_pins()
    assert caught, f"planted mistake '{name}' passed every pin"

"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function raises (AssertionError or another exception) when the
oracle disagrees with:

* the hand-computed golden blocks in tests/golden/ (layout readings of the VTE
  feature list and of the INT4 group-128 description in the datastack.it
  summary of "annotated-llm-runtime");
* IEEE-754 decoding of fp16/bf16 (checked over every finite bit pattern against
  numpy's own float16 / float32 types);
* closed forms: float32 dequantization is the exact value rounded once and does
  not depend on the order of the products; x = e_k extracts column k exactly;
* invariants: zero scale -> zero weights, weights affine in the code with slope
  d*sc, the zero point of each format;
* brute force: the float64 GEMV against an exact rational sum;
* silu against closed forms from the math module, and the SwiGLU chain on
  hand-made matrices whose GEMVs are exact integers;
* the byte counts of the decode workloads (34, 144 and 210 bytes per block)
  and of GGUF's Q5_K block (176 bytes).

They are plain functions so tests/test_oracle_mutants.py can run them against
an oracle with a planted mistake and check that some pin catches it.
"""
from fractions import Fraction

import numpy as np

import oracle
from golden_io import all_names, load
from synth import gen_weights, gen_x, rng

FMTS = ("q8_0", "q4_k", "q6_k", "int4_g128", "q5_k")
MIN_FMTS = ("q4_k", "q5_k")     # formats with a per-sub-block min term


# -- encodings ----------------------------------------------------------------
def pin_fp16_decode():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 10) & 0x1F) != 0x1F
    got = oracle.fp16_bits_to_f64(bits[finite])
    ref = bits[finite].view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    # a few values fixed by the binary16 definition itself
    table = {0x3C00: 1.0, 0x3800: 0.5, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x7BFF: 65504.0, 0xC000: -2.0, 0x3555: 0.333251953125}
    for b, v in table.items():
        assert oracle.fp16_bits_to_f64(np.uint16(b)) == v


def pin_bf16_decode():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    got = oracle.bf16_bits_to_f64(bits[finite])
    ref = (bits[finite].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, ref)
    assert oracle.bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0
    assert oracle.bf16_bits_to_f64(np.uint16(0x0001)) == 2.0 ** -133


def pin_bf16_rne():
    g = rng(7)
    x = g.standard_normal(20000).astype(np.float32)
    # exact ties: low half 0x8000 with even and odd kept bits
    tie_bits = (g.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, tie_bits.view(np.float32)[np.isfinite(tie_bits.view(np.float32))]])
    got = oracle.f32_to_bf16_bits_rne(x).astype(np.uint32)
    u = x.view(np.uint32)
    lo = u >> 16                                   # truncation toward zero (magnitude)
    hi = lo + 1
    xv = x.astype(np.float64)
    vlo = (lo << 16).view(np.float32).astype(np.float64)
    vhi = (hi << 16).view(np.float32).astype(np.float64)
    dlo, dhi = np.abs(xv - vlo), np.abs(vhi - xv)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(got, want)


# -- golden blocks ------------------------------------------------------------
def pin_golden(name):
    g = load(name)
    fmt, rows, cols = g["fmt"], g["rows"], g["cols"]
    assert g["data"].size == oracle.packed_size(fmt, rows, cols), name
    w = oracle.dequant64(fmt, g["data"], rows, cols)
    bad = np.argwhere(w != g["w"])
    assert bad.size == 0, f"{name}: first mismatch at {bad[:4].tolist()}"
    ones = np.ones((1, cols), np.float32)
    y = oracle.gemv64(fmt, g["data"], rows, cols, ones, "f32")
    for r, v in g["row_sums"]:
        assert y[0, r] == v, f"{name}: row {r} sum {y[0, r]} != {v}"
    # re-packing the decoded fields must give back the same bytes
    f = oracle.unpack(fmt, g["data"], rows, cols)
    assert np.array_equal(oracle.pack(fmt, f, rows, cols), g["data"]), name


def pin_packed_sizes():
    # bytes per block quoted with the decode workloads: Q8_0 34 B, Q4_K 144 B, Q6_K 210 B
    assert oracle.packed_size("q8_0", 1, 32) == 34
    assert oracle.packed_size("q4_k", 1, 256) == 144
    assert oracle.packed_size("q6_k", 1, 256) == 210
    assert oracle.packed_size("q5_k", 1, 256) == 176   # 2 + 2 + 12 + 32 + 128
    assert oracle.packed_size("int4_g128", 1, 128) == 64 + 2
    assert oracle.packed_size("q8_0", 1536, 1536) == 2_506_752
    assert oracle.packed_size("q4_k", 18944, 3584) == 38_191_104
    assert oracle.packed_size("q4_k", 3584, 18944) == 38_191_104
    assert oracle.packed_size("q6_k", 152064, 3584) == 447_068_160
    assert oracle.packed_size("int4_g128", 18944, 3584) == 35_008_512


# -- helpers to build fields with chosen scales --------------------------------
def _fields(fmt, rows, cols, seed, scale_bits=None):
    f = gen_weights(fmt, rows, cols, seed)
    if scale_bits is not None:
        key = "s_bits" if fmt == "int4_g128" else "d_bits"
        f[key] = np.broadcast_to(np.asarray(scale_bits, np.uint16), f[key].shape).copy()
        if fmt in MIN_FMTS:
            f["dmin_bits"] = f[key][:, ::-1].copy()
    return f


def _scale64(fmt, f):
    key = "s_bits" if fmt == "int4_g128" else "d_bits"
    return oracle.fp16_bits_to_f64(f[key])


EXTREME_SCALES = [0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xBC00, 0x8001, 0x1234]


def pin_roundtrip(fmt):
    rows, cols = 3, 2 * oracle.QK[fmt]
    for seed in range(3):
        f = _fields(fmt, rows, cols, 50 + seed)
        data = oracle.pack(fmt, f, rows, cols)
        back = oracle.unpack(fmt, data, rows, cols)
        for k, v in f.items():
            assert np.array_equal(np.asarray(back[k]).reshape(np.shape(v)), v), (fmt, k)
    # extreme codes
    f = _fields(fmt, rows, cols, 9)
    lo_hi = {"q8_0": ("q", -128, 127), "q4_k": ("u", 0, 15), "q6_k": ("q", 0, 63),
             "int4_g128": ("q", -8, 7), "q5_k": ("u", 0, 31)}[fmt]
    key, lo, hi = lo_hi
    f[key][:, ::2] = lo
    f[key][:, 1::2] = hi
    if fmt in MIN_FMTS:
        f["sc"][...] = 63
        f["m"][:, :, ::2] = 0
    back = oracle.unpack(fmt, oracle.pack(fmt, f, rows, cols), rows, cols)
    for k, v in f.items():
        assert np.array_equal(np.asarray(back[k]).reshape(np.shape(v)), v), (fmt, k)


def pin_single_rounding(fmt):
    """float32 dequant = exact value rounded once, whatever the product order."""
    rows, cols = 4, 2 * oracle.QK[fmt]
    for i, sb in enumerate([None] + EXTREME_SCALES):
        f = _fields(fmt, rows, cols, 100 + i, sb)
        data = oracle.pack(fmt, f, rows, cols)
        w64 = oracle.dequant64(fmt, data, rows, cols)
        w32 = oracle.dequant32(fmt, data, rows, cols)
        assert np.array_equal(w32, w64.astype(np.float32))
        if fmt not in MIN_FMTS:
            assert np.array_equal(w32.astype(np.float64), w64), "product must be exact in float32"
            continue
        # Q4_K / Q5_K: the two products are exact in float32, so any order gives the same result.
        nb = cols // 256
        d = oracle.fp16_bits_to_f64(f["d_bits"]).astype(np.float32)[:, :, None, None]
        dm = oracle.fp16_bits_to_f64(f["dmin_bits"]).astype(np.float32)[:, :, None, None]
        sc = f["sc"].astype(np.float32)[:, :, :, None]
        m = f["m"].astype(np.float32)[:, :, :, None]
        u = f["u"].astype(np.float32).reshape(rows, nb, 8, 32)
        order1 = (d * sc) * u - dm * m
        order2 = d * (sc * u) - m * dm
        assert np.array_equal(order1.reshape(rows, cols), w32)
        assert np.array_equal(order2.reshape(rows, cols), w32)


def pin_zero_scale(fmt):
    rows, cols = 2, 2 * oracle.QK[fmt]
    f = _fields(fmt, rows, cols, 200, 0x0000)
    if fmt in MIN_FMTS:
        f["dmin_bits"][...] = 0
    w = oracle.dequant64(fmt, oracle.pack(fmt, f, rows, cols), rows, cols)
    assert np.all(w == 0)
    if fmt in MIN_FMTS:  # d = 0 leaves only the min term
        f["dmin_bits"][...] = 0x3C00
        w = oracle.dequant64(fmt, oracle.pack(fmt, f, rows, cols), rows, cols)
        want = -np.repeat(f["m"].astype(np.float64).reshape(rows, -1), 32, axis=1)
        assert np.array_equal(w, want)


def pin_affine_in_code(fmt):
    """All codes equal to c: w(c+1) - w(c) = d*sc exactly; the format's zero point gives 0."""
    rows, cols = 2, oracle.QK[fmt]
    f = _fields(fmt, rows, cols, 300)
    key = {"q8_0": "q", "q4_k": "u", "q6_k": "q", "int4_g128": "q", "q5_k": "u"}[fmt]
    rng_c = {"q8_0": range(-128, 127), "q4_k": range(0, 15), "q6_k": range(0, 63),
             "int4_g128": range(-8, 7), "q5_k": range(0, 31)}[fmt]
    zero = {"q8_0": 0, "q6_k": 32, "int4_g128": 0}
    prev = None
    d = _scale64(fmt, f)[:, 0]
    if fmt in MIN_FMTS:
        slope = np.repeat(d[:, None] * f["sc"][:, 0, :].astype(np.float64), 32, axis=1)
    elif fmt == "q6_k":
        slope = np.repeat(d[:, None] * f["sc"][:, 0, :].astype(np.float64), 16, axis=1)
    else:
        slope = np.repeat(d[:, None], cols, axis=1)
    for c in rng_c:
        f[key][...] = c
        w = oracle.dequant64(fmt, oracle.pack(fmt, f, rows, cols), rows, cols)
        if prev is not None:
            assert np.array_equal(w - prev, slope), (fmt, c)
        if fmt in zero and c == zero[fmt]:
            assert np.all(w == 0), (fmt, c)
        if fmt in MIN_FMTS and c == 0:
            dmin = oracle.fp16_bits_to_f64(f["dmin_bits"])[:, 0]
            want = -np.repeat(dmin[:, None] * f["m"][:, 0, :].astype(np.float64), 32, axis=1)
            assert np.array_equal(w, want)
        prev = w


def pin_gemv_bruteforce(fmt):
    """Tiny non-square GEMVs: float64 result vs exact rational sum; x = e_k -> column k."""
    for rows, nblk, batch in [(3, 1, 1), (5, 2, 2), (8, 1, 3)]:
        cols = nblk * oracle.QK[fmt]
        f = _fields(fmt, rows, cols, 400 + rows)
        data = oracle.pack(fmt, f, rows, cols)
        for xd in ("f32", "f16", "bf16"):
            x = gen_x(batch, cols, xd, 500 + rows)
            y = oracle.gemv64(fmt, data, rows, cols, x, xd)
            assert y.shape == (batch, rows)
            w = oracle.dequant64(fmt, data, rows, cols)
            x64 = x64_numpy(x, xd)  # not the oracle's own decoder
            for b in range(batch):
                for r in range(rows):
                    exact = sum(Fraction(float(w[r, k])) * Fraction(float(x64[b, k]))
                                for k in range(cols))
                    assert abs(Fraction(float(y[b, r])) - exact) <= abs(exact) * Fraction(1, 10 ** 13) + Fraction(1, 10 ** 300)
        w = oracle.dequant64(fmt, data, rows, cols)
        for k in (0, cols // 2 + 1, cols - 1):
            e = np.zeros((1, cols), np.float32)
            e[0, k] = 1.0
            y = oracle.gemv64(fmt, data, rows, cols, e, "f32")
            assert np.array_equal(y[0], w[:, k])
        # sampled-row path equals the full path (up to float64 summation order)
        ids = [rows - 1, 0]
        x = gen_x(2, cols, "f32", 9)
        assert np.allclose(oracle.gemv64_rows(fmt, data, rows, cols, x, "f32", ids),
                           oracle.gemv64(fmt, data, rows, cols, x, "f32")[:, ids],
                           rtol=1e-13, atol=0)


# -- the parity gate, its diagnostic and the activation reading -----------------
def x64_numpy(x, x_dtype):
    """Exact float64 activations built from numpy's own conversions: float32 and
    float16 values widened by numpy, bf16 bits as the upper half of a binary32."""
    x = np.asarray(x)
    if x_dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def pin_x_to_f64():
    """Activation decoding per dtype against numpy's conversions, and the dtype
    deciding how the same 16 bits are read."""
    g = rng(11)
    v = (g.standard_normal(509) * 3.0).astype(np.float32)
    v[:6] = [0.0, -0.0, 6.0e-8, -65504.0, 1.0e-30, 3.0e38]
    assert np.array_equal(oracle.x_to_f64(v, "f32"), v.astype(np.float64))
    h = v[:4].copy()
    h = np.concatenate([h, v[6:]]).astype(np.float16)
    assert np.array_equal(oracle.x_to_f64(h, "f16"), h.astype(np.float64))
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.x_to_f64(bits, "bf16"),
                          (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    # 0x3C00 is 1.0 in binary16 and 2^-7 in bfloat16; 0xC0A0 is -2.3125 and -5.0
    b = np.array([0x3C00, 0x4000, 0xC0A0], np.uint16)
    assert np.array_equal(oracle.x_to_f64(b.view(np.float16), "f16"), [1.0, 2.0, -2.3125])
    assert np.array_equal(oracle.x_to_f64(b, "bf16"), [2.0 ** -7, 2.0, -5.0])
    for xd, arr in (("f32", h), ("f16", v), ("bf16", h), ("f16", bits)):
        try:
            oracle.x_to_f64(arr, xd)
        except TypeError:
            continue
        raise AssertionError(f"{xd} accepted a {arr.dtype} array")


def pin_normwise_gate():
    """The 2e-3 gate's error measure on hand-computed cases: one value per
    activation row, the largest deviation over that row's outputs divided by
    that row's largest |y64|; an all-zero reference row admits only exact
    zero; NaN and infinities fail."""
    y64 = np.array([[1.0, -4.0, 2.0], [0.5, 0.25, -1.0]])
    y = np.array([[1.5, -4.0, 2.0], [0.5, 0.5, -1.0]])
    err = oracle.normwise_rel_err(y, y64)
    assert err.shape == (2,) and err[0] == 0.125 and err[1] == 0.25   # 0.5/4, 0.25/1
    # the largest deviation, not an average: one bad output of eight
    y64 = np.ones((1, 8))
    y = y64.copy()
    y[0, 5] += 2.0 ** -4
    assert oracle.normwise_rel_err(y, y64)[0] == 2.0 ** -4
    # each activation row is scaled by its own largest |y64|
    y64 = np.array([[1000.0, 0.0], [1.0, -2.0]])
    y = np.array([[1000.0, 0.0], [1.0, -2.5]])
    assert np.array_equal(oracle.normwise_rel_err(y, y64), [0.0, 0.25])
    # all-zero reference rows
    y64 = np.zeros((2, 3))
    y = np.zeros((2, 3))
    y[1, 2] = 1e-300
    assert np.array_equal(oracle.normwise_rel_err(y, y64), [0.0, np.inf])
    assert oracle.normwise_rel_err(np.array([[-0.0, 0.0]]), np.zeros((1, 2)))[0] == 0.0
    for bad in (np.nan, np.inf, -np.inf):
        e = oracle.normwise_rel_err(np.array([[1.0, bad]]), np.array([[1.0, 2.0]]))
        assert e[0] == np.inf, bad
    # a single activation row as a 1-D vector
    assert oracle.normwise_rel_err(np.array([3.0, 4.0]), np.array([2.0, 4.0])) == 0.25


def pin_elementwise_bound():
    """gamma_{K+1} * sum_k |w x| on a hand-made row, and as an upper bound of
    float32 dot products of exact operands summed in three orders."""
    u = 2.0 ** -24
    assert oracle.gamma(33) == 33 * u / (1 - 33 * u)
    f = {"d_bits": np.array([[0x3C00]], np.uint16), "q": np.zeros((1, 32), np.int8)}
    f["q"][0, :2] = [1, -2]
    data = oracle.pack("q8_0", f, 1, 32)
    x = np.zeros((1, 32), np.float32)
    x[0, :2] = [3.0, 4.0]
    b = oracle.elementwise_bound("q8_0", data, 1, 32, x, "f32")
    assert b.shape == (1, 1) and b[0, 0] == 11.0 * oracle.gamma(33)   # |1*3| + |-2*4|
    assert np.array_equal(oracle.elementwise_bound_rows("q8_0", data, 1, 32, x, "f32", [0]), b)
    # formats whose weights are exact in float32 (one rounding per product)
    for fmt in ("q8_0", "q6_k", "int4_g128"):
        rows, cols = 6, 2 * oracle.QK[fmt]
        d = _fields(fmt, rows, cols, 610)
        data = oracle.pack(fmt, d, rows, cols)
        x = gen_x(2, cols, "f32", 611)
        w32 = oracle.dequant32(fmt, data, rows, cols)
        y64 = oracle.gemv64(fmt, data, rows, cols, x, "f32")
        bound = oracle.elementwise_bound(fmt, data, rows, cols, x, "f32")
        assert np.allclose(bound[:, [4, 1]],    # float64 summation order differs
                           oracle.elementwise_bound_rows(fmt, data, rows, cols, x, "f32", [4, 1]),
                           rtol=1e-13, atol=0)
        yb, bb = oracle.gemv64_and_bound(fmt, data, rows, cols, x, "f32", row_chunk=4)
        assert np.allclose(yb, y64, rtol=1e-13, atol=0) and np.allclose(bb, bound, rtol=1e-13, atol=0)
        for bi in range(2):
            prods = w32 * x[bi][None, :]                     # float32 products, rounded once
            seq = np.add.accumulate(prods, axis=1, dtype=np.float32)[:, -1]
            rev = np.add.accumulate(prods[:, ::-1], axis=1, dtype=np.float32)[:, -1]
            pair = prods.sum(axis=1, dtype=np.float32)
            for y32 in (seq, rev, pair):
                assert np.all(np.abs(y32.astype(np.float64) - y64[bi]) <= bound[bi]), fmt


def pin_swiglu():
    """silu against closed forms built with the math module, and the SwiGLU
    chain against hand-made Q8_0 matrices whose GEMVs are exact integers:
    h[b, r] = silu(g[b, r]) * u[b, r] with gate and up not interchangeable
    (silu(2) * 3 != silu(3) * 2), rows paired by index and batch rows apart."""
    import math
    pts = [0.0, 1.0, -1.0, 2.5, -7.0, 30.0]
    want = [p / (1.0 + math.exp(-p)) for p in pts]
    got = oracle.silu64(np.array(pts))
    assert np.allclose(got, want, rtol=1e-15, atol=0)
    assert got[0] == 0.0 and abs(got[1] - 0.7310585786300049) < 1e-15
    big = oracle.silu64(np.array([-800.0, 800.0, np.nan]))
    assert big[0] == 0.0 and np.signbit(big[0]) and big[1] == 800.0 and np.isnan(big[2])
    # gate row r has code gq[r] at column 0 and up row r has uq[r] there (d = 1),
    # so with x = (x0, 0, ..., 0): g = gq[r] * x0, u = uq[r] * x0
    rows, cols = 3, 32
    gq, uq = [2, -1, 0], [3, 5, -4]
    gf = {"d_bits": np.full((rows, 1), 0x3C00, np.uint16), "q": np.zeros((rows, cols), np.int8)}
    uf = {"d_bits": np.full((rows, 1), 0x3C00, np.uint16), "q": np.zeros((rows, cols), np.int8)}
    gf["q"][:, 0] = gq
    uf["q"][:, 0] = uq
    gd, ud = oracle.pack("q8_0", gf, rows, cols), oracle.pack("q8_0", uf, rows, cols)
    x = np.zeros((2, cols), np.float32)
    x[:, 0] = [1.0, -0.5]
    h = oracle.swiglu64("q8_0", gd, ud, rows, cols, x, "f32")
    assert h.shape == (2, rows)
    for b, x0 in enumerate((1.0, -0.5)):
        for r in range(rows):
            g, u = gq[r] * x0, uq[r] * x0
            assert abs(h[b, r] - g / (1.0 + math.exp(-g)) * u) <= 1e-15 * max(1.0, abs(g * u)), (b, r)
    assert abs(h[0, 0] - 3 * 2 / (1 + math.exp(-2))) < 1e-14        # 5.2848..., not silu(3) * 2
    # sampled rows equal the full result
    assert np.array_equal(oracle.swiglu64("q8_0", gd, ud, rows, cols, x, "f32", [2, 0]), h[:, [2, 0]])


ALL_PINS = (
    [("fp16_decode", pin_fp16_decode, ()), ("bf16_decode", pin_bf16_decode, ()),
     ("bf16_rne", pin_bf16_rne, ()), ("packed_sizes", pin_packed_sizes, ()),
     ("x_to_f64", pin_x_to_f64, ()), ("normwise_gate", pin_normwise_gate, ()),
     ("elementwise_bound", pin_elementwise_bound, ()), ("swiglu", pin_swiglu, ())]
    + [(f"golden[{n}]", pin_golden, (n,)) for n in all_names()]
    + [(f"{p.__name__[4:]}[{fmt}]", p, (fmt,)) for fmt in FMTS
       for p in (pin_roundtrip, pin_single_rounding, pin_zero_scale, pin_affine_in_code,
                 pin_gemv_bruteforce)]
)


def failing_pins():
    """Names of the pins that fail against the oracle as currently loaded."""
    bad = []
    for name, fn, args in ALL_PINS:
        try:
            fn(*args)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            bad.append(name)
    return bad

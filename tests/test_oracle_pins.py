"""Pins of the CPU oracle against what the pages and mathematics fix.

Each pin is chosen so that a plausible slip in the oracle (a swapped nibble,
a dropped min term, a transposed operand, a wrong tie rule, SiLU on the wrong
projection) fails at least one test.  Nothing here touches the GPU path.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import read_golden

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------ helpers

def f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", v))[0]


def f32_from_bits(b):
    return struct.unpack("<f", struct.pack("<I", b))[0]


def mx_block(e, codes):
    """MXFP4 block from an exponent byte and 32 codes (element 2j = high nibble)."""
    assert len(codes) == 32
    qs = [(codes[2 * j] << 4) | codes[2 * j + 1] for j in range(16)]
    return np.array([e] + qs, dtype=np.uint8)


def q2k_block(scales, qs, d_bits, dmin_bits):
    b = np.zeros(84, dtype=np.uint8)
    b[0:16] = scales
    b[16:80] = qs
    b[80:82] = np.array([d_bits], dtype="<u2").view(np.uint8)
    b[82:84] = np.array([dmin_bits], dtype="<u2").view(np.uint8)
    return b


def e2m1_golden():
    return {int(c): float(v) for c, v in read_golden("e2m1_table.txt")}


# ------------------------------------------------------------------ formats

def test_golden_geometry():
    g = {r[0]: (int(r[1]), int(r[2])) for r in read_golden("formats.txt")}
    assert g["mxfp4"] == (17, 32)
    assert g["q2k"] == (84, 256)
    assert g["int4g32"] == (18, 32)  # 16 B of codes + 2 B BF16 scale per group
    assert len(mx_block(127, [0] * 32)) == 17
    assert len(oracle.mxfp4_decode(np.zeros(17, np.uint8))) == 32
    assert len(oracle.q2k_decode(np.zeros(84, np.uint8))) == 256


def test_e2m1_table_matches_pages():
    table = e2m1_golden()
    assert len(table) == 16
    for c in range(16):
        v = oracle.e2m1(c)
        assert v == table[c], c
        assert math.copysign(1.0, v) == math.copysign(1.0, table[c]), c  # -0.0 at code 8
    for c in range(8):  # codes 8..15 are the negatives of 0..7
        assert oracle.e2m1(c + 8) == -oracle.e2m1(c)


def test_e8m0_power_of_two_and_bit_pattern():
    for e in range(0, 255):
        assert oracle.e8m0(e) == math.ldexp(1.0, e - 127), e
    # The scalar reference reinterprets e<<23 as fp32 and maps e == 0 to the
    # pattern 0x00400000; both readings give 2^-127 and 255 gives +inf.
    for e in range(1, 256):
        assert oracle.e8m0(e) == f32_from_bits(e << 23)
    assert oracle.e8m0(0) == f32_from_bits(0x00400000) == 2.0 ** -127
    assert math.isinf(oracle.e8m0(255))


def test_mxfp4_nibble_order_high_first():
    blk = np.zeros(17, np.uint8)
    blk[0] = 127
    blk[1] = 0x71  # high nibble 7 (6.0) is element 0, low nibble 1 (0.5) element 1
    w = oracle.mxfp4_decode(blk)
    assert w[0] == 6.0 and w[1] == 0.5
    assert np.all(w[2:] == 0)


def test_mxfp4_decode_all_codes_all_config_exponents():
    table = e2m1_golden()
    codes = list(range(16)) * 2
    blocks = np.stack([mx_block(e, codes) for e in range(118, 135)])
    w = oracle.mxfp4_decode(blocks).reshape(17, 32)
    for r, e in enumerate(range(118, 135)):
        for i, c in enumerate(codes):
            assert Fraction(w[r, i]) == Fraction(table[c]) * Fraction(2) ** (e - 127)


def test_mxfp4_matches_fp32_scalar_reference_form():
    # Second route to the same numbers: fp32 table value times the fp32 whose
    # bit pattern is e<<23 (the page's scalar reference), on random blocks.
    table = np.array([v for _, v in sorted(e2m1_golden().items())], dtype=np.float32)
    blocks = RNG.integers(0, 256, size=(200, 17), dtype=np.uint8)
    blocks[:, 0] = RNG.integers(1, 200, size=200)
    w = oracle.mxfp4_decode(blocks).reshape(200, 32)
    for b in range(200):
        scale = np.array([int(blocks[b, 0]) << 23], dtype=np.uint32).view(np.float32)[0]
        for j in range(16):
            hi, lo = blocks[b, 1 + j] >> 4, blocks[b, 1 + j] & 0xF
            assert w[b, 2 * j] == float(table[hi] * scale)
            assert w[b, 2 * j + 1] == float(table[lo] * scale)


def test_q2k_handbuilt_ramp():
    # scale nibble 1, min nibble 0, every qs byte 0xE4 = 0b11_10_01_00,
    # d = 1.0, dmin = 0  ->  weights 0,1,2,3 repeating (2-bit codes LSB first).
    w = oracle.q2k_decode(q2k_block([0x01] * 16, [0xE4] * 64, 0x3C00, 0x0000))
    assert list(w) == [0.0, 1.0, 2.0, 3.0] * 64


def test_q2k_handbuilt_min_term():
    # scale 0, min nibble 1, codes 0, dmin = 1.0  ->  w = -dmin*m = -1 everywhere.
    w = oracle.q2k_decode(q2k_block([0x10] * 16, [0] * 64, 0x3C00, 0x3C00))
    assert np.all(w == -1.0)
    w0 = oracle.q2k_decode(q2k_block([0x00] * 16, [0xFF] * 64, 0x3C00, 0x3C00))
    assert np.all(w0 == 0.0)


def test_q2k_subblock_scale_and_min_roles():
    # scales[j] = j (scale j, min 0), all codes 1, d = 0.5: w_i = 0.5 * (i // 16).
    w = oracle.q2k_decode(q2k_block(list(range(16)), [0x55] * 64, 0x3800, 0x0000))
    assert list(w) == [0.5 * (i // 16) for i in range(256)]
    # scale 15, min j, code 3, d = 2^-10 (0x1400), dmin = 0.25 (0x3400):
    # w_i = 2^-10 * 45 - 0.25 * (i // 16).
    w = oracle.q2k_decode(q2k_block([(j << 4) | 0xF for j in range(16)], [0xFF] * 64, 0x1400, 0x3400))
    assert list(w) == [45 * 2.0 ** -10 - 0.25 * (i // 16) for i in range(256)]


def test_q2k_code_byte_position():
    for p in (0, 5, 17, 63):
        qs = [0] * 64
        qs[p] = 0x1B  # 0b00_01_10_11: codes 3, 2, 1, 0 for weights 4p .. 4p+3
        w = oracle.q2k_decode(q2k_block([0x01] * 16, qs, 0x4000, 0x0000))  # d = 2
        expect = [0.0] * 256
        expect[4 * p:4 * p + 4] = [6.0, 4.0, 2.0, 0.0]
        assert list(w) == expect, p


def test_q2k_subnormal_f16_scale():
    w = oracle.q2k_decode(q2k_block([0x01] * 16, [0x03] * 64, 0x0001, 0x0000))  # d = 2^-24
    assert w[0] == 3 * 2.0 ** -24 and w[1] == 0.0


def test_int4_packing_and_levels():
    levels = [int(v) for v in read_golden("int4_levels.txt")[0]]
    assert levels == list(range(-8, 8))
    q = np.array([0x76543210, 0xFEDCBA98, 0x00000000, 0x7777_7777], dtype=np.uint32).view(np.int32)
    w = oracle.int4g32_decode(q, np.array([0x3F80], np.uint16))  # scale 1.0
    assert list(w[:8]) == [0, 1, 2, 3, 4, 5, 6, 7]
    assert list(w[8:16]) == [-8, -7, -6, -5, -4, -3, -2, -1]
    assert list(w[16:24]) == [0] * 8 and list(w[24:32]) == [7] * 8
    w3 = oracle.int4g32_decode(q, np.array([0x4040], np.uint16))  # scale 3.0
    assert np.all(w3 == 3 * w)
    assert sorted(set(w.tolist())) == [float(v) for v in levels]


def test_bf16_and_f16_decoders():
    assert oracle.bf16_to_float(0x3F80) == 1.0
    assert oracle.bf16_to_float(0xC040) == -3.0
    assert oracle.bf16_to_float(0x0001) == 2.0 ** -133
    assert oracle.f16_to_float(0x3C00) == 1.0
    assert oracle.f16_to_float(0x0001) == 2.0 ** -24
    assert oracle.f16_to_float(0xC000) == -2.0
    for bits in RNG.integers(0, 0x7F80, size=500):
        assert oracle.bf16_to_float(int(bits)) == f32_from_bits(int(bits) << 16)
    for bits in RNG.integers(0, 0x7C00, size=500):
        assert oracle.f16_to_float(int(bits)) == float(np.array([bits], np.uint16).view(np.float16)[0])


def test_bf16_rne_ties_and_fp32_agreement():
    assert oracle.bf16_rne(1.0) == 0x3F80
    assert oracle.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80           # tie -> even
    assert oracle.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82       # tie -> even (up)
    assert oracle.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # above the tie
    assert oracle.bf16_rne(-0.0) == 0x8000
    assert oracle.bf16_rne(1e39) == 0x7F80
    # On fp32 inputs it must agree with rounding the fp32 bit pattern.
    vals = RNG.standard_normal(2000).astype(np.float32) * np.float32(100)
    for v in vals:
        u = f32_bits(float(v))
        expect = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
        assert oracle.bf16_rne(float(v)) == expect


# ------------------------------------------------------------------ matvec

def exact_gemv(w_frac_rows, x_frac):
    return [sum((a * b for a, b in zip(row, x_frac)), Fraction(0)) for row in w_frac_rows]


def check_fp64_sum(y, exact, absterms):
    # Recursive summation bound: |fl(sum) - sum| <= gamma_K * sum|terms|.
    K = len(absterms[0]) if isinstance(absterms[0], list) else 1
    for yi, ei, at in zip(y, exact, absterms):
        k = len(at)
        gamma = k * 2.0 ** -53 / (1 - k * 2.0 ** -53)
        bound = gamma * float(sum(at))
        assert abs(Fraction(yi) - ei) <= Fraction(bound) + Fraction(1, 10 ** 300), (yi, float(ei))
    return K


@pytest.mark.parametrize("n,k", [(64, 64), (3, 96), (5, 32)])
def test_gemv_mxfp4_brute_force_exact(n, k):
    blocks = RNG.integers(0, 256, size=(n * k // 32, 17), dtype=np.uint8)
    blocks[:, 0] = RNG.integers(118, 135, size=blocks.shape[0])
    x = RNG.standard_normal((2, k)).astype(np.float32)
    y = oracle.gemv("mxfp4", blocks, n, k, x.astype(np.float64))
    table = e2m1_golden()
    rows = []
    for r in range(n):
        row = []
        for b in range(k // 32):
            blk = blocks[r * (k // 32) + b]
            sc = Fraction(2) ** (int(blk[0]) - 127)
            for j in range(16):
                row.append(Fraction(table[blk[1 + j] >> 4]) * sc)
                row.append(Fraction(table[blk[1 + j] & 0xF]) * sc)
        rows.append(row)
    for t in range(2):
        xf = [Fraction(float(v)) for v in x[t]]
        ex = exact_gemv(rows, xf)
        check_fp64_sum(y[t], ex, [[abs(a * b) for a, b in zip(row, xf)] for row in rows])


def test_gemv_mxfp4_integer_special_case_matches_int64_matmul():
    # e = 127 and codes {0,2,4,5,6,7} give the integers {0,1,2,3,4,6}; with
    # integer activations the fp64 sums are exact and equal an int64 matmul.
    n, k = 64, 64
    allowed = np.array([0, 2, 4, 5, 6, 7])
    value = {0: 0, 2: 1, 4: 2, 5: 3, 6: 4, 7: 6}
    codes = allowed[RNG.integers(0, 6, size=(n, k))]
    blocks = np.stack([mx_block(127, list(codes[r, 32 * b:32 * b + 32]))
                       for r in range(n) for b in range(k // 32)])
    x = RNG.integers(-50, 51, size=(3, k))
    y = oracle.gemv("mxfp4", blocks, n, k, x.astype(np.float64))
    wi = np.vectorize(value.get)(codes).astype(np.int64)
    assert np.array_equal(y, (x.astype(np.int64) @ wi.T).astype(np.float64))


def test_gemv_single_nonzero_locates_row_and_column():
    n, k = 7, 96
    blocks = np.zeros((n * k // 32, 17), np.uint8)
    blocks[:, 0] = 127
    r0, k0 = 5, 70                       # weight (5, 70): block 2 of row 5, element 6
    blk = blocks[r0 * 3 + k0 // 32]
    blk[1 + (k0 % 32) // 2] = 0x70       # element 6 is the high nibble of byte 3: code 7 = 6.0
    x = np.zeros(k)
    x[k0] = 2.0
    x[k0 + 1] = 1000.0                   # the neighbouring element must not leak in
    y = oracle.gemv("mxfp4", blocks, n, k, x)[0]
    expect = np.zeros(n)
    expect[r0] = 12.0
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("n,k", [(64, 256), (4, 512)])
def test_gemv_q2k_brute_force_exact(n, k):
    nb = n * k // 256
    blocks = RNG.integers(0, 256, size=(nb, 84), dtype=np.uint8)
    d = (RNG.uniform(1e-3, 1e-2, size=(nb, 2))).astype(np.float16)
    blocks[:, 80:84] = d.view(np.uint8).reshape(nb, 4)
    x = RNG.standard_normal((1, k)).astype(np.float32)
    y = oracle.gemv("q2k", blocks, n, k, x.astype(np.float64))[0]
    rows = []
    for r in range(n):
        row = []
        for b in range(k // 256):
            blk = blocks[r * (k // 256) + b]
            dd = Fraction(float(blk[80:82].view(np.float16)[0]))
            dm = Fraction(float(blk[82:84].view(np.float16)[0]))
            for i in range(256):
                s = blk[i // 16]
                q = (int(blk[16 + i // 4]) >> (2 * (i % 4))) & 3
                row.append(dd * (s & 0xF) * q - dm * (s >> 4))
        rows.append(row)
    xf = [Fraction(float(v)) for v in x[0]]
    check_fp64_sum(y, exact_gemv(rows, xf), [[abs(a * b) for a, b in zip(row, xf)] for row in rows])


def test_gemv_int4_brute_force_exact():
    n, k = 64, 64
    q = RNG.integers(-2 ** 31, 2 ** 31, size=(n, k // 8), dtype=np.int64).astype(np.int32)
    s = RNG.integers(0x3C00, 0x4000, size=(n, k // 32)).astype(np.uint16)
    x = RNG.standard_normal((2, k)).astype(np.float32)
    y = oracle.gemv("int4g32", (q, s), n, k, x.astype(np.float64))
    rows = []
    for r in range(n):
        row = []
        for i in range(k):
            word = int(q[r, i // 8]) & 0xFFFFFFFF
            v = (word >> (4 * (i % 8))) & 0xF
            v = v - 16 if v >= 8 else v
            row.append(v * Fraction(f32_from_bits(int(s[r, i // 32]) << 16)))
        rows.append(row)
    for t in range(2):
        xf = [Fraction(float(v)) for v in x[t]]
        check_fp64_sum(y[t], exact_gemv(rows, xf), [[abs(a * b) for a, b in zip(row, xf)] for row in rows])


# ------------------------------------------------------------------ routing

def test_router_logits_exact_on_small_case():
    E, D = 8, 64
    wr = RNG.standard_normal((E, D)).astype(np.float32)
    x = RNG.standard_normal((2, D)).astype(np.float32).astype(np.float64)
    lg = oracle.router_logits(wr, x)
    for t in range(2):
        for e in range(E):
            terms = [Fraction(float(a)) * Fraction(float(b)) for a, b in zip(wr[e], x[t])]
            ex = sum(terms, Fraction(0))
            gamma = D * 2.0 ** -53 / (1 - D * 2.0 ** -53)
            assert abs(Fraction(lg[t, e]) - ex) <= Fraction(gamma * float(sum(abs(v) for v in terms)))


def test_topk_ties_resolve_to_lower_index():
    E, D = 256, 64
    wr = (RNG.standard_normal((E, D)) * 0.01).astype(np.float32)
    big = np.abs(RNG.standard_normal(D)).astype(np.float32)
    for e in (40, 10, 200):
        wr[e] = big                      # three identical rows with the largest logits
    x = np.ones((1, D), dtype=np.float64)
    idx, g = oracle.topk_softmax(oracle.router_logits(wr, x), 6)
    assert list(idx[0, :3]) == [10, 40, 200]
    assert g[0, 0] == g[0, 1] == g[0, 2]


def test_topk_zero_activation_gives_first_six_uniform():
    wr = RNG.standard_normal((256, 64)).astype(np.float32)
    idx, g = oracle.topk_softmax(oracle.router_logits(wr, np.zeros((1, 64))), 6)
    assert list(idx[0]) == [0, 1, 2, 3, 4, 5]
    assert np.all(g[0] == 1.0 / 6.0)


def test_topk_matches_stable_argsort_and_softmax_closed_form():
    logits = RNG.standard_normal((50, 256)) * 3.0
    logits[7, 100] = logits[7, 3] = 50.0      # an exact tie at the top
    idx, g = oracle.topk_softmax(logits, 6)
    for t in range(50):
        ref = np.argsort(-logits[t], kind="stable")[:6]
        assert list(idx[t]) == list(ref)
        sel = logits[t, ref]
        ex = [math.exp(v - sel[0]) for v in sel]
        tot = math.fsum(ex)
        for j in range(6):
            assert abs(g[t, j] - ex[j] / tot) <= 4e-16
        assert abs(math.fsum(g[t]) - 1.0) <= 1e-15
        assert np.all(np.diff(g[t]) <= 0)
    assert list(idx[7, :2]) == [3, 100]


# ------------------------------------------------------------------ FFN / layer

def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == 1.0 / (1.0 + math.exp(-1.0))
    assert oracle.silu(-1.0) == -1.0 / (1.0 + math.e)
    assert oracle.silu(1000.0) == 1000.0
    s = oracle.silu(-1000.0)
    assert s == 0.0 and math.copysign(1.0, s) == -1.0


def _rand_mx(n, k, rng):
    b = rng.integers(0, 256, size=(n * k // 32, 17), dtype=np.uint8)
    b[:, 0] = rng.integers(118, 135, size=b.shape[0])
    return b.reshape(-1)


def test_layer_identical_experts_reduce_to_one_expert():
    rng = np.random.default_rng(7)
    E, D, F = 16, 64, 32
    gate, up, down = _rand_mx(F, D, rng), _rand_mx(F, D, rng), _rand_mx(D, F, rng)
    wr = (rng.standard_normal((E, D)) * 0.02).astype(np.float32)
    x = (rng.standard_normal((1, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y, idx, g = oracle.layer_decode("mxfp4", lambda e: (gate, up, down), wr, x, 6, F)
    one = oracle.expert_ffn("mxfp4", gate, up, down, oracle.bf16_rows_to_f64(x), D, F)
    assert np.allclose(y, one, rtol=1e-12, atol=0)
    assert abs(g.sum() - 1.0) < 1e-15


def test_layer_identical_tokens_identical_rows():
    rng = np.random.default_rng(8)
    E, D, F = 16, 64, 32
    experts = [(_rand_mx(F, D, rng), _rand_mx(F, D, rng), _rand_mx(D, F, rng)) for _ in range(E)]
    wr = (rng.standard_normal((E, D)) * 0.02).astype(np.float32)
    x1 = (rng.standard_normal((1, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = np.repeat(x1, 4, axis=0)
    y, idx, g = oracle.layer_decode("mxfp4", lambda e: experts[e], wr, x, 6, F)
    assert all(np.array_equal(y[0], y[t]) for t in range(4))
    assert all(np.array_equal(idx[0], idx[t]) for t in range(4))


def _silu_ref(z):
    # z * sigmoid(z); e^-z overflows for z < -709, where the product is -0.
    if z < -700.0:
        return -0.0
    return z / (1.0 + math.exp(-z))


def test_layer_brute_force_tiny():
    # Exact-rational gate/up/down with SiLU evaluated in double on the exact
    # gate value: checks which projection is gated, the gating product, the
    # down projection and the slot-weighted combine.
    rng = np.random.default_rng(9)
    E, D, F, K = 8, 64, 32, 2
    experts = [(_rand_mx(F, D, rng), _rand_mx(F, D, rng), _rand_mx(D, F, rng)) for _ in range(E)]
    wr = (rng.standard_normal((E, D)) * 0.05).astype(np.float32)
    xb = (rng.standard_normal((2, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y, idx, g = oracle.layer_decode("mxfp4", lambda e: experts[e], wr, xb, K, F)
    xf = oracle.bf16_rows_to_f64(xb)

    def rows(blocks, n, k):
        w = oracle.mxfp4_decode(blocks).reshape(n, k)   # decode itself is pinned above
        return [[Fraction(float(v)) for v in r] for r in w]

    for t in range(2):
        xfr = [Fraction(float(v)) for v in xf[t]]
        acc = [Fraction(0)] * D
        for j in range(K):
            gt, upw, dn = experts[int(idx[t, j])]
            gv = exact_gemv(rows(gt, F, D), xfr)
            uv = exact_gemv(rows(upw, F, D), xfr)
            h = [Fraction(_silu_ref(float(a))) * b for a, b in zip(gv, uv)]
            yp = exact_gemv(rows(dn, D, F), h)
            acc = [a + Fraction(float(g[t, j])) * b for a, b in zip(acc, yp)]
        ref = np.array([float(v) for v in acc])
        assert np.max(np.abs(y[t] - ref)) <= 1e-9 * np.max(np.abs(ref))


def test_rmsnorm_closed_forms():
    D = 64
    h = np.full((1, D), 3.0)
    # mean(h^2) = 9: x = bf16(3 / sqrt(9 + 1e-6)) = bf16(0.99999994...) = 1.0
    assert np.all(oracle.rmsnorm_bf16(h) == 0x3F80)
    h = np.zeros((1, D))
    h[0, 0] = 8.0                        # mean = 1, x0 = bf16(8/sqrt(1+1e-6)) = 8.0
    out = oracle.rmsnorm_bf16(h)
    assert out[0, 0] == 0x4100 and np.all(out[0, 1:] == 0)
    h = RNG.standard_normal((3, D)) * 1e11
    out = oracle.bf16_array_to_f64(oracle.rmsnorm_bf16(h))
    rms = np.sqrt(np.mean(h ** 2, axis=1, keepdims=True))
    assert np.allclose(out, h / rms, rtol=2 ** -8)



# ------------------------------------------------------------------ stack

def _tiny_stack(n_layers, seed, zero_down=False):
    rng = np.random.default_rng(seed)
    E, D, F = 8, 64, 32
    experts = []
    for _ in range(n_layers):
        lay = []
        for _ in range(E):
            g, u, d = _rand_mx(F, D, rng), _rand_mx(F, D, rng), _rand_mx(D, F, rng)
            if zero_down:
                d = d.reshape(-1, 17).copy()
                d[:, 1:] = 0          # every code 0: the down projection is the zero matrix
                d = d.reshape(-1)
            lay.append((g, u, d))
        experts.append(lay)
    routers = [(rng.standard_normal((E, D)) * 0.05).astype(np.float32) for _ in range(n_layers)]
    h0 = (rng.standard_normal((3, D)) * 2.0).astype(np.float32)
    return experts, routers, h0, F


def test_stack_zero_updates_keep_the_residual():
    experts, routers, h0, F = _tiny_stack(3, 31, zero_down=True)
    h = oracle.stack_decode("mxfp4", lambda l, e: experts[l][e], routers, h0, 2, F)
    assert np.array_equal(h, h0.astype(np.float64))


def test_stack_norm_hides_a_power_of_two_scale():
    # With eps = 0 the norm of 4 h equals the norm of h exactly, so layer 0
    # sees the same activation and adds the same update to the scaled state.
    experts, routers, h0, F = _tiny_stack(1, 32)
    get = lambda l, e: experts[l][e]
    h_a, (step_a,) = oracle.stack_decode("mxfp4", get, routers, h0, 2, F, eps=0.0, trace=True)
    h4 = (h0 * np.float32(4.0)).astype(np.float32)
    h_b, (step_b,) = oracle.stack_decode("mxfp4", get, routers, h4, 2, F, eps=0.0, trace=True)
    assert np.array_equal(step_a[0], step_b[0]) and np.any(step_a[0] != 0)
    assert np.array_equal(step_a[3], step_b[3])
    assert np.array_equal(h_b, h4.astype(np.float64) + step_a[3])
    assert not np.array_equal(h_a, h_b)


def test_stack_equals_explicit_norm_layer_residual_chain():
    experts, routers, h0, F = _tiny_stack(2, 33)
    h, steps = oracle.stack_decode("mxfp4", lambda l, e: experts[l][e], routers, h0, 2, F, trace=True)
    cur = h0.astype(np.float64)
    for l in range(2):
        x = oracle.rmsnorm_bf16(cur, 1e-6)
        y, idx, g = oracle.layer_decode("mxfp4", lambda e, _l=l: experts[_l][e], routers[l], x, 2, F)
        assert np.array_equal(x, steps[l][0]) and np.array_equal(idx, steps[l][1])
        cur = cur + y
    assert np.array_equal(h, cur)


# ------------------------------------------------------------------ FP4 -> INT4

def test_int4_candidates_from_pages():
    cands = [Fraction(int(a), int(b)) for a, b in read_golden("int4_candidates.txt")]
    ours = oracle.int4_candidates()
    assert len(ours) == 6
    for c, o in zip(cands, ours):
        # each is the fp32 nearest to the page's number (a float32 tensor times a Python float)
        assert o == float(np.float32(float(c)))


def _quant_one(e, codes):
    q, s, s_f, r = oracle.quantize_fp4_to_int4g32(mx_block(e, codes), 1, 32, with_detail=True)
    w = oracle.int4g32_decode(q, s)
    word_codes = []
    for wi in range(4):
        word = int(q[0, wi]) & 0xFFFFFFFF
        for i in range(8):
            v = (word >> (4 * i)) & 0xF
            word_codes.append(v - 16 if v >= 8 else v)
    return word_codes, int(s[0, 0]), float(s_f[0, 0]), int(r[0, 0]), w


def test_int4_worked_example_all_sixes():
    # All weights 6.0: r = 1.0 reproduces them exactly (q = 7, s = 6/7); every
    # earlier candidate has s < 6/7 and clips 6 to 7*s < 6, so r = 1.0 wins.
    codes, scale, s, r, _ = _quant_one(127, [7] * 32)
    assert codes == [7] * 32 and r == 3
    assert s == float(np.float32(6.0) / np.float32(7.0))
    assert scale == 0x3F5B
    codes, scale, s, r, _ = _quant_one(127, [15] * 32)   # all -6.0
    assert codes == [-7] * 32 and r == 3 and scale == 0x3F5B


def test_int4_worked_example_all_zero_takes_first_candidate():
    # amax clamps to 1e-8; every candidate gives q = 0 and zero error, and only
    # a strictly smaller error replaces the best, so r = 6/7 (the first) wins.
    codes, scale, s, r, _ = _quant_one(127, [0] * 32)
    assert codes == [0] * 32 and r == 0
    amax = np.float32(1e-8)
    assert s == float((amax * np.float32(6.0 / 7.0)) / np.float32(7.0))
    assert scale == 0x30A8


def _exact_argmin(w):
    """Brute force with exact rational errors over the six fp32 scales."""
    w32 = np.array(w, dtype=np.float32)
    amax = max(np.float32(np.max(np.abs(w32))), np.float32(1e-8))
    best = None
    for j, (a, b) in enumerate(read_golden("int4_candidates.txt")):
        r32 = np.float32(int(a) / int(b))
        s = np.float32(np.float32(amax * r32) / np.float32(7.0))
        q = np.clip(np.rint(w32 / s), -8, 7).astype(int)
        err = sum((Fraction(float(wi)) - int(qi) * Fraction(float(s))) ** 2 for wi, qi in zip(w32, q))
        if best is None or err < best[0]:
            best = (err, j, float(s), list(q))
    return best


def test_int4_worked_examples_mixed_blocks():
    # One 6.0 among 31 x 0.5 and the 16 codes twice: checked against the exact
    # brute force, and against the values derived from it.
    codes, scale, s, r, _ = _quant_one(127, [7] + [1] * 31)
    err, j, s_ref, q_ref = _exact_argmin([6.0] + [0.5] * 31)
    assert (r, s, codes) == (j, s_ref, q_ref)
    assert r == 0 and codes == [7] + [1] * 31 and scale == 0x3F3C

    ramp = list(range(16)) * 2
    codes, scale, s, r, _ = _quant_one(127, ramp)
    err, j, s_ref, q_ref = _exact_argmin([oracle.e2m1(c) for c in ramp])
    assert (r, s, codes) == (j, s_ref, q_ref)
    assert r == 2 and scale == 0x3F50
    assert codes == [0, 1, 1, 2, 2, 4, 5, 7, 0, -1, -1, -2, -2, -4, -5, -7] * 2
    codes130, scale130, s130, r130, _ = _quant_one(130, ramp)
    assert codes130 == codes and r130 == r and s130 == 8 * s and scale130 == 0x40D0


def test_int4_random_blocks_match_exact_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(300):
        e = int(rng.integers(118, 135))
        codes = [int(c) for c in rng.integers(0, 16, size=32)]
        got_codes, _, s, r, _ = _quant_one(e, codes)
        w = [oracle.e2m1(c) * 2.0 ** (e - 127) for c in codes]
        _, j, s_ref, q_ref = _exact_argmin(w)
        assert (r, s, got_codes) == (j, s_ref, q_ref)


def test_int4_scale_invariance_and_rounding_properties():
    rng = np.random.default_rng(12)
    n = 400
    blocks = rng.integers(0, 256, size=(n, 17), dtype=np.uint8)
    blocks[:, 0] = 120
    q0, s0, sf0, r0 = oracle.quantize_fp4_to_int4g32(blocks, n, 32, with_detail=True)
    blocks2 = blocks.copy()
    blocks2[:, 0] = 131
    q1, s1, sf1, r1 = oracle.quantize_fp4_to_int4g32(blocks2, n, 32, with_detail=True)
    assert np.array_equal(q0, q1) and np.array_equal(r0, r1)
    assert np.array_equal(sf1, sf0 * np.float32(2.0 ** 11))
    # bf16 of an exact power-of-two multiple only shifts the exponent field
    assert np.array_equal(s1.astype(np.int32), s0.astype(np.int32) + (11 << 7))
    w = oracle.mxfp4_decode(blocks).reshape(n, 32)
    wq = oracle.int4g32_decode(q0, s0).reshape(n, 32)
    for i in range(n):
        s = float(sf0[i, 0])
        qv = wq[i] / oracle.bf16_to_float(int(s0[i, 0]))
        assert np.all((qv >= -8) & (qv <= 7))
        inside = np.abs(w[i] / s) <= 7.5
        assert np.all(np.abs(w[i][inside] - qv[inside] * s) <= s / 2 * (1 + 1e-6))
        # never worse than the plain r = 1 quantiser
        amax = np.float32(np.max(np.abs(w[i])))
        s1_ = np.float32(np.float32(amax * np.float32(1.0)) / np.float32(7.0))
        qq = np.clip(np.rint(w[i].astype(np.float32) / s1_), -8, 7).astype(np.float64)
        e_plain = np.sum((w[i] - qq * np.float64(s1_)) ** 2)
        e_best = np.sum((w[i] - qv * s) ** 2)
        assert e_best <= e_plain * (1 + 1e-12)


# ---------------------------------------------------------------- hash-routed layers

def test_hash_route_closed_form():
    """Experts come from the table row in its order; the weights are the
    softmax of their logits: logits ln(1..8) give weights proportional to
    the chosen experts' 1+index ("cabbage v4x quant surgery", hash layers)."""
    l = np.log(np.arange(1, 9, dtype=np.float64))[None, :]
    table = np.array([[7, 0, 2], [1, 3, 5]], dtype=np.int32)
    idx, g, nb = oracle.hash_route(l, 3, table, np.array([0], dtype=np.int32))
    assert nb == 0 and idx.tolist() == [[7, 0, 2]]
    np.testing.assert_allclose(g[0], np.array([8.0, 1.0, 3.0]) / 12.0, rtol=1e-15)
    idx, g, _ = oracle.hash_route(np.vstack([l, l + 50.0]), 3, table, np.array([1, 1], dtype=np.int32))
    assert idx.tolist() == [[1, 3, 5], [1, 3, 5]]
    np.testing.assert_allclose(g[1], g[0], rtol=1e-14)   # softmax: a common shift changes nothing
    np.testing.assert_allclose(g[0], np.array([2.0, 4.0, 6.0]) / 12.0, rtol=1e-15)


def test_hash_route_equals_learned_route_on_its_own_choice():
    """A table row that holds a token's learned top-k (in rank order) gives
    exactly the learned routing's weights (same shift, same order): a check
    against the independent top-k routine."""
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((5, 40))
    idx_l, g_l = oracle.topk_softmax(logits, 6)
    table = idx_l.astype(np.int32)                      # vocab 5: token id b -> row b
    idx_h, g_h, nb = oracle.hash_route(logits, 6, table, np.arange(5, dtype=np.int32))
    assert nb == 0
    assert np.array_equal(idx_h, idx_l)
    assert np.array_equal(g_h, g_l)


def test_hash_route_invalid_ids_and_rows():
    l = np.zeros((4, 16))
    table = np.array([[3, 4, 5], [3, 3, 5], [3, 16, 5]], dtype=np.int32)
    idx, g, nb = oracle.hash_route(l, 3, table, np.array([0, 1, 2, 7], dtype=np.int32))
    assert nb == 3                                       # repeated expert, expert >= E, id >= vocab
    assert idx.tolist() == [[3, 4, 5], [0, 1, 2], [0, 1, 2], [0, 1, 2]]
    np.testing.assert_allclose(g, 1.0 / 3.0, rtol=1e-15)


def test_hashed_layer_composition():
    """A hash-routed layer is the learned layer's expert FFN and combine with
    the table's experts: with a table holding the learned choice it gives the
    learned layer's result exactly."""
    rng = np.random.default_rng(13)
    E, D, F, k = 6, 64, 64, 2
    experts = {e: (_rand_mx(F, D, rng), _rand_mx(F, D, rng), _rand_mx(D, F, rng)) for e in range(E)}
    wr = (rng.standard_normal((E, D)) * 0.05).astype(np.float32)
    xb = (rng.standard_normal((1, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    _, _, logits = oracle.route_topk(wr, xb, k)
    learned_idx, _ = oracle.topk_softmax(logits, k)
    table = learned_idx.astype(np.int32)
    y_h, i_h, g_h = oracle.layer_decode("mxfp4", lambda e: experts[e], wr, xb, k, F,
                                        hashed=(table, np.array([0], dtype=np.int32)))
    y_l, i_l, g_l = oracle.layer_decode("mxfp4", lambda e: experts[e], wr, xb, k, F)
    assert np.array_equal(i_h, i_l) and np.array_equal(g_h, g_l) and np.array_equal(y_h, y_l)


# ---------------------------------------------------------------- alternative numerics
# "ds4.c study notes", glossary page "quantization": "MXFP4's ROCm native
# kernel" (Q8_K activations, integer dots) and "Metal's MXFP4 -> half lookup
# table" (exactly rounded binary16 products).

def test_q8k_quantize_closed_forms():
    k = np.arange(-127, 128)
    x = np.concatenate([k * 0.5, [0.0]]).astype(np.float32).reshape(1, 256)  # max |x| = 63.5: d = 0.5 exactly
    q, d = oracle.q8k_quantize(x)
    assert d[0, 0] == np.float32(0.5)
    assert np.array_equal(q[0, :255], k) and q[0, 255] == 0
    x = np.zeros((1, 256), np.float32)
    x[0, :4] = [127.0, 2.5, 3.5, -2.5]  # d = 1: ties go to the even integer
    q, d = oracle.q8k_quantize(x)
    assert d[0, 0] == 1.0 and list(q[0, :4]) == [127, 2, 4, -2]
    x = np.zeros((2, 512), np.float32)
    x[1, 300] = -5.0
    q, d = oracle.q8k_quantize(x)
    assert np.all(d[0] == 0) and np.all(q[0] == 0) and d[1, 0] == 0  # a block of zeros: d = 0, q = 0
    assert d[1, 1] == np.float32(5.0) / np.float32(127.0) and q[1, 300] == -127


def test_q8k_quantize_error_bound():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((3, 1024)) * np.exp(rng.uniform(-4, 4, size=(3, 1)))).astype(np.float32)
    q, d = oracle.q8k_quantize(x)
    dd = np.repeat(d.astype(np.float64), 256, axis=1)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(np.abs(x.astype(np.float64) - dd * q) <= dd * (0.5 + 127 * 2.0 ** -23))
    assert np.all(np.abs(q).reshape(3, 4, 256).max(axis=2) == 127)  # each block's largest value maps to +-127


def test_gemv_mxfp4_q8_integer_route_matches_float_route():
    rng = np.random.default_rng(12)
    N, K = 24, 768
    blocks = _rand_mx(N, K, rng)
    x = rng.standard_normal((3, K)).astype(np.float32)
    q, d = oracle.q8k_quantize(x)
    y, a = oracle.gemv_mxfp4_q8(blocks, N, K, q, d)
    xd = q.astype(np.float64) * np.repeat(d.astype(np.float64), 256, axis=1)  # exact
    y2 = oracle.gemv("mxfp4", blocks, N, K, xd)
    assert np.all(np.abs(y - y2) <= 1e-13 * a)


def test_gemv_mxfp4_q8_handbuilt():
    # scale byte 128 (x2) and code 1 (0.5): every weight is 1; q = 1 with d = 0.25 -> y = K / 4
    K = 512
    blocks = np.concatenate([mx_block(128, [1] * 32) for _ in range(K // 32)])
    q = np.ones((1, K), np.int8)
    d = np.full((1, K // 256), 0.25, np.float32)
    y, a = oracle.gemv_mxfp4_q8(blocks, 1, K, q, d)
    assert y[0, 0] == K / 4 and a[0, 0] == K / 4
    # code 15 (-6) in the high nibble of byte 0 only: element 0, the first activation
    codes = [0] * 32
    codes[0] = 15
    blocks = np.concatenate([mx_block(127, codes)] + [mx_block(127, [0] * 32) for _ in range(K // 32 - 1)])
    q = np.zeros((1, K), np.int8)
    q[0, 0], q[0, 1] = 3, 100
    y, _ = oracle.gemv_mxfp4_q8(blocks, 1, K, q, np.full((1, K // 256), 1.0, np.float32))
    assert y[0, 0] == -18.0


def test_mxfp4_half_lut_matches_independent_rounding():
    lut = oracle.mxfp4_half_lut()
    for e in range(255):
        exact = np.array([oracle.e2m1(c) * 2.0 ** (e - 127) for c in range(16)], dtype=np.float64)
        with np.errstate(over="ignore"):
            ref = exact.astype(np.float16).view(np.uint16)  # numpy's binary64 -> binary16, ties to even
        assert np.array_equal(lut[e], ref), e
    assert np.all(lut[255] == 0x7E00)
    row = np.array([oracle.e2m1(c) for c in range(16)], dtype=np.float16).view(np.uint16)
    assert np.array_equal(lut[127], row)  # scale 1: the E2M1 table itself


def test_mxfp4_half_lut_golden():
    import hashlib
    rows = read_golden("mxfp4_half_lut.txt")
    lut = oracle.mxfp4_half_lut()
    sha = [r[1] for r in rows if r[0] == "sha256"][0]
    assert hashlib.sha256(lut.astype("<u2").tobytes()).hexdigest() == sha
    for r in rows:
        if r[0] == "entry":
            assert lut[int(r[1]), int(r[2])] == int(r[3], 16), r


def test_gemv_mxfp4_half_equals_exact_decode_in_range():
    # scale bytes 118..134 keep every product a normal binary16: the table
    # decode is then exact and the matvec equals the plain one
    rng = np.random.default_rng(13)
    N, K = 16, 256
    blocks = _rand_mx(N, K, rng)
    x = rng.standard_normal((2, K))
    assert np.array_equal(oracle.gemv_mxfp4_half(blocks, N, K, x), oracle.gemv("mxfp4", blocks, N, K, x))
    # out of range: scale byte 150 turns every nonzero weight into an infinity
    big = blocks.copy().reshape(-1, 17)
    big[:, 0] = 150
    y = oracle.gemv_mxfp4_half(big.reshape(-1), N, K, np.abs(x) + 1.0)
    assert np.all(np.isinf(y) | np.isnan(y))

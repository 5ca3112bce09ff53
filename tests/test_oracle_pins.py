"""Pins for the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a library routine, the mathematics
(closed forms, exact rational arithmetic on tiny inputs) or an invariant of the
definition, chosen so that a plausible slip in the oracle (a dropped chunk, a
wrong sign, a transposed operand, a wrong scale index, rounding through FP32)
fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E4M3_ONE = 0x38          # 1.0 in OCP e4m3
NAN_BYTES = (0x7F, 0xFF)


def _valid_bytes(rng, shape):
    """Random e4m3 bytes with the two NaN codes removed."""
    b = rng.integers(0, 256, size=shape, dtype=np.uint8)
    b[b == 0x7F] = 0x7E
    b[b == 0xFF] = 0xFE
    return b


def _torch_dec(byte_array):
    t = torch.from_numpy(np.ascontiguousarray(byte_array, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---- element codecs ---------------------------------------------------------

def test_dec_all_256_bytes_match_torch_float8_e4m3fn():
    ref = _torch_dec(np.arange(256, dtype=np.uint8))
    got = np.array([oracle.dec_e4m3(i) for i in range(256)])
    nan_ref = np.isnan(ref)
    assert list(np.nonzero(nan_ref)[0]) == list(NAN_BYTES)
    assert np.array_equal(np.isnan(got), nan_ref)
    assert np.array_equal(got[~nan_ref], ref[~nan_ref])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x80] == 0.0


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def test_bf16_rne_matches_torch_on_fp32_exact_inputs():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties and near-ties: low 16 bits exactly 0x8000 / 0x7FFF / 0x8001
    base = rng.integers(0, 2 ** 16, size=3000, dtype=np.uint32) << 16
    ties = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001]).astype(np.uint32)
    xt = ties.view(np.float32)
    xt = xt[np.isfinite(xt)]
    x = np.concatenate([x, xt, np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.4e38, 1e-40, -1e-45])])
    want = _torch_bf16_bits(x)
    got = np.array([oracle.bf16_rne(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("value,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                   # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),               # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),      # above the tie: direct rounding goes up;
                                                 # rounding through FP32 first would tie down
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
    (2.0 ** -134, 0x0000),                       # half the smallest subnormal: tie -> 0
    (3 * 2.0 ** -134, 0x0002),                   # tie between 1 and 2 subnormal units -> 2
    (2.0 ** -133, 0x0001),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),      # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),      # tie above the largest finite -> inf
    (2.0 ** 200, 0x7F80),
    (-0.0, 0x8000),
])
def test_bf16_rne_special_cases(value, bits):
    assert oracle.bf16_rne(value) == bits


# ---- exact rational arithmetic on tiny inputs --------------------------------

def _exact_bf16(q: Fraction) -> int:
    """Round an exact rational to BF16 bits, nearest, ties to even (independent of the C code)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e - 7, -133)
    n = a / (Fraction(2) ** quantum_exp)
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = Fraction(fl) * Fraction(2) ** quantum_exp
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(v))      # exact: at most 8 significant bits
    return sign | int((int(np.array(f).view(np.uint32)) >> 16) & 0x7FFF)


def _exact_value(Aq, SA, Bq, SB, r, n, g=0):
    """Exact rational value of one output, decoding through torch's float8 type."""
    K = Aq.shape[-1]
    a = [Fraction(float(v)) for v in _torch_dec(Aq[r])]
    b = [Fraction(float(v)) for v in _torch_dec(Bq[g][n])]
    total = Fraction(0)
    for c in range(K // 128):
        pc = sum(a[k] * b[k] for k in range(128 * c, 128 * c + 128))
        total += pc * Fraction(float(SA[r][c])) * Fraction(float(SB[g][n // 128][c]))
    return total


def _near_midpoint(q: Fraction, rel=2.0 ** -40) -> bool:
    """True if q lies within rel (relative) of a BF16 rounding midpoint."""
    if q == 0:
        return False
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 7, -133)
    n = a / quantum
    frac = n - (n.numerator // n.denominator)
    return abs(frac - Fraction(1, 2)) * quantum <= a * Fraction(rel)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 128, 0), (2, 3, 256, 1), (3, 2, 256, 2),
                                        (3, 3, 128, 3)])
def test_brute_force_exact_rationals(M, N, K, seed):
    rng = np.random.default_rng(100 + seed)
    Aq = _valid_bytes(rng, (M, K))
    Bq = _valid_bytes(rng, (1, N, K))
    SA = rng.uniform(1e-4, 3.0, size=(M, K // 128)).astype(np.float32)
    SB = rng.uniform(1e-4, 3.0, size=(1, (N + 127) // 128, K // 128)).astype(np.float32)
    D = oracle.dense(Aq, SA, Bq[0], SB[0])
    for r in range(M):
        for n in range(N):
            q = _exact_value(Aq, SA, Bq, SB, r, n)
            want = _exact_bf16(q)
            if D[r, n] != want:
                assert _near_midpoint(q), (r, n, hex(D[r, n]), hex(want), float(q))


# ---- closed forms ------------------------------------------------------------

def test_constant_inputs_give_k_a_b():
    M, N, K = 4, 200, 7168
    A = np.full((M, K), E4M3_ONE, dtype=np.uint8)
    B = np.full((N, K), E4M3_ONE, dtype=np.uint8)
    SA = np.ones((M, K // 128), np.float32)
    SB = np.ones(((N + 127) // 128, K // 128), np.float32)
    D = oracle.dense(A, SA, B, SB)
    assert np.all(D == 0x45E0)               # 7168 = 1.75 * 2^12, exact in BF16
    # a = 2 (0x40), b = -0.5 (0xB0), sa = 2^-3, sb = 4: K * a * b * sa * sb = -3584
    A[:] = 0x40
    B[:] = 0xB0
    SA[:] = 0.125
    SB[:] = 4.0
    D = oracle.dense(A, SA, B, SB)
    assert _exact_bf16(Fraction(-3584)) == 0xC560
    assert np.all(D == 0xC560)


def test_power_of_two_scales_pin_scale_indexing():
    """A = B = 1.0; SA[r][c] = 2^(r-c), SB[j][c] = 2^(j+3c).
    D[r][n] = 128 * 2^(r + n//128) * sum_c 4^c, exact in BF16 for K/128 <= 4."""
    M, N, K = 6, 3 * 128 + 40, 512
    kb = K // 128
    A = np.full((M, K), E4M3_ONE, dtype=np.uint8)
    B = np.full((N, K), E4M3_ONE, dtype=np.uint8)
    SA = np.array([[2.0 ** (r - c) for c in range(kb)] for r in range(M)], np.float32)
    nb = (N + 127) // 128
    SB = np.array([[2.0 ** (j + 3 * c) for c in range(kb)] for j in range(nb)], np.float32)
    D = oracle.dense(A, SA, B, SB)
    geo = sum(4 ** c for c in range(kb))
    for r in range(M):
        for n in range(N):
            want = _exact_bf16(Fraction(128 * geo) * Fraction(2) ** (r + n // 128))
            assert D[r, n] == want, (r, n)


def test_one_hot_rows_pin_operand_addressing():
    """Row r of A is 1.0 at k = pi(r) and 0 elsewhere; scales are powers of two.
    Then D[r][n] = dec(B[n][pi(r)]) * SA[r][pi(r)//128] * SB[n//128][pi(r)//128] exactly."""
    rng = np.random.default_rng(7)
    M, N, K = 9, 300, 640
    kb, nb = K // 128, (N + 127) // 128
    A = np.zeros((M, K), np.uint8)
    pi = rng.choice(K, size=M, replace=False)
    A[np.arange(M), pi] = E4M3_ONE
    B = _valid_bytes(rng, (N, K))
    SA = (2.0 ** rng.integers(-4, 5, size=(M, kb))).astype(np.float32)
    SB = (2.0 ** rng.integers(-4, 5, size=(nb, kb))).astype(np.float32)
    D = oracle.dense(A, SA, B, SB)
    Bv = _torch_dec(B)
    for r in range(M):
        c = pi[r] // 128
        for n in range(N):
            v = Fraction(float(Bv[n, pi[r]])) * Fraction(float(SA[r, c])) * Fraction(float(SB[n // 128, c]))
            assert D[r, n] == _exact_bf16(v), (r, n)


def test_zero_a_gives_zero():
    rng = np.random.default_rng(3)
    M, N, K = 3, 130, 256
    A = np.zeros((M, K), np.uint8)
    B = _valid_bytes(rng, (N, K))
    SA = rng.uniform(0.1, 2, size=(M, 2)).astype(np.float32)
    SB = rng.uniform(0.1, 2, size=(2, 2)).astype(np.float32)
    D = oracle.dense(A, SA, B, SB)
    assert np.all((D == 0) | (D == 0x8000))


def test_chunk_sums_equal_float64_library_matmul():
    """Each chunk sum is exact in FP64, so a library FP64 matmul per 128-K chunk gives
    the same P_c; with the same FP64 promotion order the pre-rounding values agree
    bit for bit (a transposed operand or a wrong chunk/scale index breaks this)."""
    rng = np.random.default_rng(5)
    M, N, K = 17, 300, 512
    kb, nb = K // 128, (N + 127) // 128
    A = _valid_bytes(rng, (M, K))
    B = _valid_bytes(rng, (N, K))
    SA = rng.uniform(1e-3, 2, size=(M, kb)).astype(np.float32)
    SB = rng.uniform(1e-3, 2, size=(nb, kb)).astype(np.float32)
    Af, Bf = _torch_dec(A), _torch_dec(B)
    acc = np.zeros((M, N))
    col_block = np.arange(N) // 128
    for c in range(kb):
        P = Af[:, 128 * c:128 * c + 128] @ Bf[:, 128 * c:128 * c + 128].T
        s = SA[:, c].astype(np.float64)[:, None] * SB[col_block, c].astype(np.float64)[None, :]
        acc = acc + P * s
    rr, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    got_acc, got_d = oracle.points(A, SA, B, SB, rr.ravel(), np.zeros(M * N, np.int64), nn.ravel())
    assert np.array_equal(got_acc, acc.ravel())
    assert np.array_equal(got_d, oracle.dense(A, SA, B, SB).ravel())


# ---- invariants ----------------------------------------------------------------

def _double_e4m3(byte):
    """Byte whose e4m3 value is exactly twice the input's, or None if not representable."""
    s, e, m = byte & 0x80, (byte >> 3) & 15, byte & 7
    if e == 0:                                  # subnormal m * 2^-9
        return s | (2 * m) if 2 * m < 8 else s | (1 << 3) | (2 * m - 8)
    if e + 1 > 15 or (e + 1 == 15 and m == 7):
        return None
    return s | ((e + 1) << 3) | m


def test_scale_shift_invariance_is_bit_exact():
    rng = np.random.default_rng(9)
    M, N, K = 8, 260, 512
    kb, nb = K // 128, (N + 127) // 128
    # bytes in a range where doubling stays exact and finite (exponent field <= 13)
    A = rng.integers(0, 0x70, size=(M, K), dtype=np.uint8)
    A |= (rng.integers(0, 2, size=(M, K), dtype=np.uint8) << 7)
    B = _valid_bytes(rng, (N, K))
    SA = rng.uniform(0.01, 2, size=(M, kb)).astype(np.float32)
    SB = rng.uniform(0.01, 2, size=(nb, kb)).astype(np.float32)
    D0 = oracle.dense(A, SA, B, SB)
    for (r, c) in [(0, 0), (3, 2), (7, 3)]:
        A2, SA2 = A.copy(), SA.copy()
        doubled = [_double_e4m3(int(b)) for b in A2[r, 128 * c:128 * c + 128]]
        assert all(d is not None for d in doubled)
        A2[r, 128 * c:128 * c + 128] = doubled
        assert np.array_equal(_torch_dec(A2[r, 128 * c:128 * c + 128]),
                              2 * _torch_dec(A[r, 128 * c:128 * c + 128]))
        SA2[r, c] = SA[r, c] / 2
        assert np.array_equal(oracle.dense(A2, SA2, B, SB), D0)


def test_contiguous_equals_dense_per_segment_and_leaves_padding():
    rng = np.random.default_rng(21)
    G, N, K = 3, 200, 256
    kb, nb = K // 128, (N + 127) // 128
    counts = [130, 0, 77]
    layout = np.concatenate([np.r_[np.full(c, g), np.full((-c) % 128, -1)] for g, c in
                             enumerate(counts)]).astype(np.int32)
    layout[-3] = 7           # an index >= G is treated as padding
    M = layout.size
    A = _valid_bytes(rng, (M, K))
    SA = rng.uniform(0.01, 2, size=(M, kb)).astype(np.float32)
    B = _valid_bytes(rng, (G, N, K))
    SB = rng.uniform(0.01, 2, size=(G, nb, kb)).astype(np.float32)
    D = np.full((M, N), 0x7FC1, np.uint16)
    oracle.contiguous(A, SA, B, SB, layout, D)
    for g in range(G):
        rows = np.nonzero(layout == g)[0]
        if rows.size == 0:
            continue
        Dg = oracle.dense(A[rows], SA[rows], B[g], SB[g])
        assert np.array_equal(D[rows], Dg)
    pad = (layout < 0) | (layout >= G)
    assert np.all(D[pad] == 0x7FC1)


def test_contiguous_segment_permutation_permutes_rows():
    rng = np.random.default_rng(22)
    G, N, K = 2, 140, 128
    A = _valid_bytes(rng, (256, K))
    SA = rng.uniform(0.1, 2, size=(256, 1)).astype(np.float32)
    B = _valid_bytes(rng, (G, N, K))
    SB = rng.uniform(0.1, 2, size=(G, 2, 1)).astype(np.float32)
    lay = np.r_[np.zeros(128), np.ones(128)].astype(np.int32)
    D1 = np.zeros((256, N), np.uint16)
    oracle.contiguous(A, SA, B, SB, lay, D1)
    perm = np.r_[np.arange(128, 256), np.arange(0, 128)]
    D2 = np.zeros((256, N), np.uint16)
    oracle.contiguous(A[perm], SA[perm], B, SB, lay[perm], D2)
    assert np.array_equal(D2, D1[perm])


def test_masked_equals_dense_on_valid_rows_and_leaves_the_rest():
    rng = np.random.default_rng(23)
    G, max_m, N, K = 4, 40, 150, 256
    kb, nb = K // 128, (N + 127) // 128
    masked_m = np.array([0, 40, 13, 99], np.int32)        # 99 > max_m is clamped
    A = _valid_bytes(rng, (G, max_m, K))
    SA = rng.uniform(0.01, 2, size=(G, max_m, kb)).astype(np.float32)
    B = _valid_bytes(rng, (G, N, K))
    SB = rng.uniform(0.01, 2, size=(G, nb, kb)).astype(np.float32)
    D = np.full((G, max_m, N), 0x7FC1, np.uint16)
    oracle.masked(A, SA, B, SB, masked_m, D)
    for g in range(G):
        v = min(max(int(masked_m[g]), 0), max_m)
        if v:
            assert np.array_equal(D[g, :v], oracle.dense(A[g, :v], SA[g, :v], B[g], SB[g]))
        assert np.all(D[g, v:] == 0x7FC1)


def test_points_agree_with_full_computation():
    rng = np.random.default_rng(24)
    M, N, K = 20, 270, 384
    kb, nb = K // 128, (N + 127) // 128
    A = _valid_bytes(rng, (M, K))
    SA = rng.uniform(0.01, 2, size=(M, kb)).astype(np.float32)
    B = _valid_bytes(rng, (N, K))
    SB = rng.uniform(0.01, 2, size=(nb, kb)).astype(np.float32)
    D = oracle.dense(A, SA, B, SB)
    rows = rng.integers(0, M, 500)
    cols = rng.integers(0, N, 500)
    _, d = oracle.points(A, SA, B, SB, rows, np.zeros(500, np.int64), cols)
    assert np.array_equal(d, D[rows, cols])


def test_rejects_k_not_multiple_of_128():
    A = np.zeros((2, 200), np.uint8)
    B = np.zeros((3, 200), np.uint8)
    with pytest.raises(ValueError):
        oracle.dense(A, np.ones((2, 1), np.float32), B, np.ones((1, 1), np.float32))


def test_addend_reduces_to_the_plain_product_plus_c():
    """D = C + A B^T: with C = 0 it is the plain product; with C = -(the FP64 product) it is
    zero wherever that product is exactly representable as FP32; and in general it is the
    FP64 sum of C and the exact product, rounded once (checked against the points entry)."""
    from moe_grouped_gemm_block_amd import synth
    p = synth.make_dense(40, 70, 384, seed=21)
    D0 = oracle.dense(p.A, p.SA, p.B[0], p.SB[0])
    Dz = np.zeros_like(D0)
    oracle.with_addend("dense", p.A, p.SA, p.B[0], p.SB[0], np.zeros((40, 70), np.float32), Dz)
    assert np.array_equal(Dz, D0)
    rng = np.random.default_rng(22)
    C = (rng.standard_normal((40, 70)) * 10).astype(np.float32)
    Dc = np.zeros_like(D0)
    oracle.with_addend("dense", p.A, p.SA, p.B[0], p.SB[0], C, Dc)
    rows, cols = np.meshgrid(np.arange(40), np.arange(70), indexing="ij")
    acc, _ = oracle.points(p.A, p.SA, p.B[0], p.SB[0], rows.ravel(), np.zeros(40 * 70, np.int64),
                           cols.ravel())
    want = np.array([oracle.bf16_rne(float(c) + float(a)) for c, a in zip(C.ravel(), acc)],
                    dtype=np.uint16).reshape(40, 70)
    assert np.array_equal(Dc, want)
    # masked: invalid rows untouched, valid rows as dense per slot
    q = synth.make_masked(2, 24, 70, 256, seed=23, masked_m=[5, 24])
    Cm = rng.standard_normal((2, 24, 70)).astype(np.float32)
    Dm = np.full((2, 24, 70), 0x7FC1, np.uint16)
    oracle.with_addend("masked", q.A, q.SA, q.B, q.SB, Cm, Dm, q.masked_m)
    assert np.all(Dm[0, 5:] == 0x7FC1)
    for g in range(2):
        ref = np.zeros((24, 70), np.uint16)
        oracle.with_addend("dense", q.A[g], q.SA[g], q.B[g], q.SB[g], Cm[g], ref)
        v = int(min(q.masked_m[g], 24))
        assert np.array_equal(Dm[g, :v], ref[:v])

"""Pins for the oracle's stored-form (nt / nn / tn / tt) and K-grouped products, checked
against things other than the oracle's own code:

* exact rational arithmetic on tiny inputs (written here, decoding through torch's
  float8 type), rounded exactly to BF16 / FP32;
* the invariant that the stored form does not change the value: every form equals
  the nt oracle (pinned on its own) on the same logical operands;
* closed forms: one-hot operands, constant operands with power-of-two scales, empty
  groups;
* the scale-shift invariant of one (feature, 128-token chunk) scale.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E4M3_ONE = 0x38


def _valid_bytes(rng, shape):
    b = rng.integers(0, 256, size=shape, dtype=np.uint8)
    b[b == 0x7F] = 0x7E
    b[b == 0xFF] = 0xFE
    return b


def _dec(byte_array):
    t = torch.from_numpy(np.ascontiguousarray(byte_array, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _exact_round(q: Fraction, sig_bits: int, min_exp: int, max_exp: int) -> Fraction:
    """Nearest value with sig_bits significant bits (ties to even), quantum >= 2^min_exp;
    returns +-inf (as None) past 2^(max_exp+1)."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - (sig_bits - 1), min_exp)
    n = a / Fraction(2) ** qe
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = Fraction(fl) * Fraction(2) ** qe
    if v >= Fraction(2) ** (max_exp + 1):
        return None
    return v if q > 0 else -v


def _exact_bf16_bits(q: Fraction) -> int:
    v = _exact_round(q, 8, -133, 127)
    if v is None:
        return 0x7F80 | (0x8000 if q < 0 else 0)
    f = np.float32(float(v))                       # exact: 8 significant bits
    bits = int(np.array(f).view(np.uint32)) >> 16
    if v == 0 and q < 0:
        bits |= 0x8000
    return bits


def _exact_f32(q: Fraction) -> np.float32:
    v = _exact_round(q, 24, -149, 127)
    if v is None:
        return np.float32(np.inf if q > 0 else -np.inf)
    return np.float32(float(v))                    # exact: 24 significant bits


def _near_tie(q: Fraction, sig_bits: int, min_exp: int, rel=2.0 ** -40) -> bool:
    if q == 0:
        return False
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - (sig_bits - 1), min_exp)
    n = a / quantum
    frac = n - (n.numerator // n.denominator)
    return abs(frac - Fraction(1, 2)) * quantum <= a * Fraction(rel)


def _logical(ab, A_st, B_st):
    """Logical A [M][K] and B [N][K] from the stored forms."""
    A = A_st if ab[0] == "n" else A_st.T
    B = B_st if ab[1] == "t" else B_st.T
    return np.ascontiguousarray(A), np.ascontiguousarray(B)


def _stored(ab, A, B):
    A_st = A if ab[0] == "n" else A.T
    B_st = B if ab[1] == "t" else B.T
    return np.ascontiguousarray(A_st), np.ascontiguousarray(B_st)


# ---- stored forms -----------------------------------------------------------

@pytest.mark.parametrize("ab", ["nt", "nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K,seed,with_c", [(1, 2, 128, 0, False), (3, 2, 256, 1, True),
                                                (2, 3, 256, 2, False)])
def test_layouts_brute_force_exact_rationals(ab, M, N, K, seed, with_c):
    rng = np.random.default_rng(300 + seed)
    A = _valid_bytes(rng, (M, K))
    B = _valid_bytes(rng, (N, K))
    SA = rng.uniform(1e-3, 3.0, size=(M, K // 128)).astype(np.float32)
    SB = rng.uniform(1e-3, 3.0, size=((N + 127) // 128, K // 128)).astype(np.float32)
    C = rng.standard_normal((M, N)).astype(np.float32) * 50 if with_c else None
    A_st, B_st = _stored(ab, A, B)
    D = oracle.dense_layout(ab, A_st, SA, B_st, SB, C)
    Av, Bv = _dec(A), _dec(B)
    for r in range(M):
        for n in range(N):
            q = Fraction(float(C[r, n])) if with_c else Fraction(0)
            for c in range(K // 128):
                pc = sum(Fraction(float(Av[r, k])) * Fraction(float(Bv[n, k]))
                         for k in range(128 * c, 128 * c + 128))
                q += pc * Fraction(float(SA[r, c])) * Fraction(float(SB[n // 128, c]))
            want = _exact_bf16_bits(q)
            if D[r, n] != want:
                assert _near_tie(q, 8, -133), (ab, r, n, hex(D[r, n]), hex(want))


@pytest.mark.parametrize("ab", ["nn", "tn", "tt"])
def test_every_stored_form_equals_the_nt_oracle(ab):
    rng = np.random.default_rng(310)
    M, N, K = 37, 260, 640                         # ragged scale block, M != N != K
    A = _valid_bytes(rng, (M, K))
    B = _valid_bytes(rng, (N, K))
    SA = rng.uniform(1e-3, 2, size=(M, K // 128)).astype(np.float32)
    SB = rng.uniform(1e-3, 2, size=(3, K // 128)).astype(np.float32)
    want = oracle.dense(A, SA, B, SB)
    A_st, B_st = _stored(ab, A, B)
    assert np.array_equal(oracle.dense_layout(ab, A_st, SA, B_st, SB), want)
    assert np.array_equal(oracle.dense_layout("nt", A, SA, B, SB), want)


@pytest.mark.parametrize("ab", ["nt", "nn", "tn", "tt"])
def test_one_hot_pins_the_stored_addressing(ab):
    """Logical row r of A is 1.0 at k = pi(r): D[r][n] = dec(B[n][pi(r)]) sa sb exactly."""
    rng = np.random.default_rng(320)
    M, N, K = 7, 150, 384
    kb = K // 128
    A = np.zeros((M, K), np.uint8)
    pi = rng.choice(K, size=M, replace=False)
    A[np.arange(M), pi] = E4M3_ONE
    B = _valid_bytes(rng, (N, K))
    SA = (2.0 ** rng.integers(-3, 4, size=(M, kb))).astype(np.float32)
    SB = (2.0 ** rng.integers(-3, 4, size=(2, kb))).astype(np.float32)
    A_st, B_st = _stored(ab, A, B)
    D = oracle.dense_layout(ab, A_st, SA, B_st, SB)
    Bv = _dec(B)
    for r in range(M):
        c = pi[r] // 128
        for n in range(N):
            v = Fraction(float(Bv[n, pi[r]])) * Fraction(float(SA[r, c])) * \
                Fraction(float(SB[n // 128, c]))
            assert D[r, n] == _exact_bf16_bits(v), (ab, r, n)


# ---- K-grouped ------------------------------------------------------------------

def _kg_inputs(rng, ks, M, N):
    K = int(sum(ks))
    A = _valid_bytes(rng, (K, M))
    B = _valid_bytes(rng, (K, N))
    SA = rng.uniform(1e-3, 3.0, size=(M, K // 128)).astype(np.float32)
    SB = rng.uniform(1e-3, 3.0, size=(N, K // 128)).astype(np.float32)
    return A, SA, B, SB


@pytest.mark.parametrize("ks,M,N,seed,with_c", [([128, 0, 256], 2, 3, 0, False),
                                                ([256, 128], 3, 2, 1, True),
                                                ([0, 128], 1, 1, 2, True)])
def test_k_grouped_brute_force_exact_rationals(ks, M, N, seed, with_c):
    rng = np.random.default_rng(400 + seed)
    A, SA, B, SB = _kg_inputs(rng, ks, M, N)
    G = len(ks)
    C = (rng.standard_normal((G, M, N)) * 30).astype(np.float32) if with_c else None
    D = oracle.k_grouped(A, SA, B, SB, ks, C)
    Av, Bv = _dec(A), _dec(B)
    k0 = 0
    for g in range(G):
        for m in range(M):
            for n in range(N):
                q = Fraction(float(C[g, m, n])) if with_c else Fraction(0)
                for c in range(k0 // 128, (k0 + ks[g]) // 128):
                    pc = sum(Fraction(float(Av[k, m])) * Fraction(float(Bv[k, n]))
                             for k in range(128 * c, 128 * c + 128))
                    q += pc * Fraction(float(SA[m, c])) * Fraction(float(SB[n, c]))
                want = _exact_f32(q)
                if D[g, m, n] != want:
                    assert _near_tie(q, 24, -149), (g, m, n, D[g, m, n], want)
        k0 += ks[g]


def test_k_grouped_constant_operands_and_empty_groups():
    """A = 2, B = -0.5, SA = 2^-3, SB = 4 everywhere: D[g] = ks[g] * (-1) / 2 exactly;
    an empty group gives C (or zeros)."""
    ks = [256, 0, 384, 128]
    M, N = 5, 9
    K = sum(ks)
    A = np.full((K, M), 0x40, np.uint8)
    B = np.full((K, N), 0xB0, np.uint8)
    SA = np.full((M, K // 128), 0.125, np.float32)
    SB = np.full((N, K // 128), 4.0, np.float32)
    D = oracle.k_grouped(A, SA, B, SB, ks)
    for g, k in enumerate(ks):
        assert np.all(D[g] == np.float32(-k * 0.5)), g
    C = np.random.default_rng(1).standard_normal((4, M, N)).astype(np.float32)
    Dc = oracle.k_grouped(A, SA, B, SB, ks, C)
    assert np.array_equal(Dc[1], C[1])
    assert np.array_equal(Dc[0], (C[0].astype(np.float64) - 128.0).astype(np.float32))


def test_k_grouped_power_of_two_scales_pin_scale_indexing():
    """A = B = 1.0; SA[m][c] = 2^(m - c), SB[n][c] = 2^(2n + c): group g's value is
    128 * 2^(m + 2n) * (number of its chunks), each chunk contributing 2^(m + 2n)."""
    ks = [128, 256, 0, 384]
    M, N = 4, 3
    K = sum(ks)
    kb = K // 128
    A = np.full((K, M), E4M3_ONE, np.uint8)
    B = np.full((K, N), E4M3_ONE, np.uint8)
    SA = np.array([[2.0 ** (m - c) for c in range(kb)] for m in range(M)], np.float32)
    SB = np.array([[2.0 ** (2 * n + c) for c in range(kb)] for n in range(N)], np.float32)
    D = oracle.k_grouped(A, SA, B, SB, ks)
    for g, k in enumerate(ks):
        for m in range(M):
            for n in range(N):
                assert D[g, m, n] == np.float32(k * 2.0 ** (m + 2 * n)), (g, m, n)
    # a per-chunk pattern that tells the chunks apart: SB[n][c] = 4^c
    SB2 = np.array([[4.0 ** c for c in range(kb)] for _ in range(N)], np.float32)
    SA2 = np.ones((M, kb), np.float32)
    D2 = oracle.k_grouped(A, SA2, B, SB2, ks)
    c0 = 0
    for g, k in enumerate(ks):
        want = sum(128 * 4.0 ** c for c in range(c0, c0 + k // 128))
        assert np.all(D2[g] == np.float32(want)), g
        c0 += k // 128


def test_k_grouped_one_hot_tokens_pin_operand_addressing():
    """Feature m of A is 1.0 at one token pi(m) of group g(m): D[g][m][n] =
    dec(B[pi(m)][n]) * SA[m][c] * SB[n][c] for that group, zero for the others."""
    rng = np.random.default_rng(430)
    ks = [256, 128, 384]
    M, N = 6, 40
    K = sum(ks)
    kb = K // 128
    A = np.zeros((K, M), np.uint8)
    pi = rng.choice(K, size=M, replace=False)
    A[pi, np.arange(M)] = E4M3_ONE
    B = _valid_bytes(rng, (K, N))
    SA = (2.0 ** rng.integers(-3, 4, size=(M, kb))).astype(np.float32)
    SB = (2.0 ** rng.integers(-3, 4, size=(N, kb))).astype(np.float32)
    D = oracle.k_grouped(A, SA, B, SB, ks)
    starts = np.cumsum([0] + ks)
    Bv = _dec(B)
    for m in range(M):
        g = int(np.searchsorted(starts, pi[m], side="right") - 1)
        c = pi[m] // 128
        for gg in range(len(ks)):
            for n in range(N):
                want = (Fraction(float(Bv[pi[m], n])) * Fraction(float(SA[m, c])) *
                        Fraction(float(SB[n, c]))) if gg == g else Fraction(0)
                assert D[gg, m, n] == _exact_f32(want), (gg, m, n)


def _double_e4m3(byte):
    s, e, m = byte & 0x80, (byte >> 3) & 15, byte & 7
    if e == 0:
        return s | (2 * m) if 2 * m < 8 else s | (1 << 3) | (2 * m - 8)
    if e + 1 > 15 or (e + 1 == 15 and m == 7):
        return None
    return s | ((e + 1) << 3) | m


def test_k_grouped_scale_shift_invariance_is_bit_exact():
    rng = np.random.default_rng(440)
    ks = [256, 128]
    M, N = 5, 7
    K = sum(ks)
    B = _valid_bytes(rng, (K, N))
    A = rng.integers(0, 0x70, size=(K, M), dtype=np.uint8)
    A |= (rng.integers(0, 2, size=(K, M), dtype=np.uint8) << 7)
    SA = rng.uniform(0.01, 2, size=(M, K // 128)).astype(np.float32)
    SB = rng.uniform(0.01, 2, size=(N, K // 128)).astype(np.float32)
    D0 = oracle.k_grouped(A, SA, B, SB, ks)
    for (m, c) in [(0, 0), (3, 1), (4, 2)]:
        A2, SA2 = A.copy(), SA.copy()
        A2[128 * c:128 * c + 128, m] = [_double_e4m3(int(b)) for b in A[128 * c:128 * c + 128, m]]
        SA2[m, c] = SA[m, c] / 2
        assert np.array_equal(oracle.k_grouped(A2, SA2, B, SB, ks), D0)
    # and the same on the B side (swap the operands' roles)
    B2 = rng.integers(0, 0x70, size=(K, N), dtype=np.uint8)
    D1 = oracle.k_grouped(A, SA, B2, SB, ks)
    B3, SB3 = B2.copy(), SB.copy()
    B3[128:256, 2] = [_double_e4m3(int(b)) for b in B2[128:256, 2]]
    SB3[2, 1] = SB[2, 1] / 2
    assert np.array_equal(oracle.k_grouped(A, SA, B3, SB3, ks), D1)


def test_k_grouped_rejects_bad_group_sizes():
    A = np.zeros((256, 2), np.uint8)
    B = np.zeros((256, 2), np.uint8)
    S = np.ones((2, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.k_grouped(A, S, B, S, [100, 156])
    with pytest.raises(ValueError):
        oracle.k_grouped(A, S, B, S, [128, 256])

"""CPU oracle for the block-scaled FP8 GEMM -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the oracle never
imports the product path.

The arithmetic lives in ``fp8bs_oracle.c`` (plain C, FP64, OpenMP over output
rows); this module only builds it with gcc and marshals numpy arrays into it.
All arrays are in the oracle's *logical* layouts:

  A   uint8  [rows][K]            OCP e4m3 bytes, row-major
  SA  f32    [rows][K/128]        one scale per row and 128-wide K group
  B   uint8  [G][N][K] or [N][K]  OCP e4m3 bytes, one row per output column
  SB  f32    [G][ceil(N/128)][K/128]
  D   uint16 [rows][N]            BF16 bit patterns

The quantisers (``quant_1x128``, ``quant_128x128``) produce A/SA and B/SB in
these layouts from FP32 inputs.  ``dense_layout`` takes A and B in any of the four
stored forms nt / nn / tn / tt; ``k_grouped`` is the K-grouped (weight-gradient)
product with A [K_total][M], B [K_total][N], SA [M][K_total/128], SB [N][K_total/128]
and FP32 output D [G][M][N].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8bs_oracle.c")
_LIB = os.path.join(_HERE, "libfp8bs_oracle.so")
# A test of the pins themselves points this at a deliberately broken build.
_LIB_OVERRIDE = os.environ.get("FP8BS_ORACLE_LIB")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, -O2, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.fp8bs_oracle_dec_e4m3.argtypes = [ctypes.c_uint8]
    lib.fp8bs_oracle_dec_e4m3.restype = ctypes.c_double
    lib.fp8bs_oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.fp8bs_oracle_bf16_rne.restype = ctypes.c_uint16
    lib.fp8bs_oracle_dense.argtypes = [P, P, P, P, P, I64, I64, I64]
    lib.fp8bs_oracle_contiguous.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64]
    lib.fp8bs_oracle_masked.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64]
    lib.fp8bs_oracle_points.argtypes = [P, P, P, P, I64, I64, I64, P, P, P, P, P]
    for f in ("dense", "contiguous", "masked", "points"):
        getattr(lib, "fp8bs_oracle_" + f).restype = ctypes.c_int
    lib.fp8bs_oracle_num_threads.restype = ctypes.c_int
    lib.fp8bs_oracle_with_addend.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, I64, I64, I64, I64]
    lib.fp8bs_oracle_with_addend.restype = ctypes.c_int
    lib.fp8bs_oracle_enc_e4m3.argtypes = [ctypes.c_float]
    lib.fp8bs_oracle_enc_e4m3.restype = ctypes.c_uint8
    lib.fp8bs_oracle_quant_1x128.argtypes = [P, P, P, I64, I64]
    lib.fp8bs_oracle_quant_1x128.restype = ctypes.c_int
    lib.fp8bs_oracle_quant_128x128.argtypes = [P, P, P, I64, I64, I64]
    lib.fp8bs_oracle_quant_128x128.restype = ctypes.c_int
    lib.fp8bs_oracle_dense_layout.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P, P,
                                              I64, I64, I64]
    lib.fp8bs_oracle_dense_layout.restype = ctypes.c_int
    lib.fp8bs_oracle_k_grouped.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64]
    lib.fp8bs_oracle_k_grouped.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def num_threads() -> int:
    return int(_load().fp8bs_oracle_num_threads())


def dec_e4m3(byte: int) -> float:
    return float(_load().fp8bs_oracle_dec_e4m3(int(byte)))


def bf16_rne(x: float) -> int:
    return int(_load().fp8bs_oracle_bf16_rne(float(x)))


def _check(rc: int):
    if rc != 0:
        raise ValueError("oracle rejected the shape (K must be a positive multiple of 128)")


def dense(A, SA, B, SB, D=None):
    """D[M][N] (BF16 bits).  D, if given, is updated in place (every row is valid)."""
    A, SA, B, SB = _u8(A), _f32(SA), _u8(B), _f32(SB)
    M, K = A.shape
    N = B.shape[-2]
    if D is None:
        D = np.zeros((M, N), dtype=np.uint16)
    _check(_load().fp8bs_oracle_dense(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K))
    return D


def contiguous(A, SA, B, SB, layout, D):
    """Writes the valid rows of D[M][N] in place; padding rows keep their bits."""
    A, SA, B, SB, layout = _u8(A), _f32(SA), _u8(B), _f32(SB), _i32(layout)
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    assert D.dtype == np.uint16 and D.shape == (M, N) and D.flags["C_CONTIGUOUS"]
    _check(_load().fp8bs_oracle_contiguous(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(layout),
                                           _ptr(D), M, N, K, G))
    return D


def masked(A, SA, B, SB, masked_m, D):
    """A[G][max_m][K]; writes the valid rows of D[G][max_m][N] in place."""
    A, SA, B, SB, masked_m = _u8(A), _f32(SA), _u8(B), _f32(SB), _i32(masked_m)
    G, max_m, K = A.shape
    N = B.shape[1]
    assert D.dtype == np.uint16 and D.shape == (G, max_m, N) and D.flags["C_CONTIGUOUS"]
    _check(_load().fp8bs_oracle_masked(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(masked_m),
                                       _ptr(D), G, max_m, N, K))
    return D


def points(A, SA, B, SB, a_row, group, col):
    """Sampled outputs.  A/SA may be [rows][K] or [G][max_m][K] (flattened to rows);
    B is [N][K] or [G][N][K].  Returns (acc_fp64, d_bf16_bits)."""
    A, SA, B, SB = _u8(A), _f32(SA), _u8(B), _f32(SB)
    K = A.shape[-1]
    N = B.shape[-2]
    a_row = np.ascontiguousarray(a_row, dtype=np.int64)
    group = np.ascontiguousarray(group, dtype=np.int64)
    col = np.ascontiguousarray(col, dtype=np.int64)
    n = a_row.shape[0]
    assert group.shape == (n,) and col.shape == (n,)
    rows = A.size // K
    G = 1 if B.ndim == 2 else B.shape[0]
    if n and (a_row.min() < 0 or a_row.max() >= rows or group.min() < 0 or group.max() >= G
              or col.min() < 0 or col.max() >= N):
        raise IndexError("oracle point out of range")
    acc = np.zeros(n, dtype=np.float64)
    d = np.zeros(n, dtype=np.uint16)
    _check(_load().fp8bs_oracle_points(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), N, K, n,
                                       _ptr(a_row), _ptr(group), _ptr(col), _ptr(acc), _ptr(d)))
    return acc, d


def enc_e4m3(x: float) -> int:
    """Nearest OCP e4m3 code (ties to even) of an FP32 value of magnitude <= 448."""
    return int(_load().fp8bs_oracle_enc_e4m3(float(x)))


def quant_1x128(X):
    """X float32 [rows][K] -> (Q uint8 [rows][K], S float32 [rows][K/128])."""
    X = _f32(X)
    rows, K = X.shape
    Q = np.zeros((rows, K), dtype=np.uint8)
    S = np.zeros((rows, max(K // 128, 0)), dtype=np.float32)
    _check(_load().fp8bs_oracle_quant_1x128(_ptr(X), _ptr(Q), _ptr(S), rows, K))
    return Q, S


def quant_128x128(X):
    """X float32 [G][N][K] -> (Q uint8 [G][N][K], S float32 [G][ceil(N/128)][K/128])."""
    X = _f32(X)
    G, N, K = X.shape
    Q = np.zeros((G, N, K), dtype=np.uint8)
    S = np.zeros((G, (N + 127) // 128, max(K // 128, 0)), dtype=np.float32)
    _check(_load().fp8bs_oracle_quant_128x128(_ptr(X), _ptr(Q), _ptr(S), G, N, K))
    return Q, S


def with_addend(kind, A, SA, B, SB, C, D, gdata=None):
    """D = bf16(C + A B^T) at valid rows, D updated in place.  kind: "dense" (A [M][K],
    B [N][K] or [1][N][K]), "contiguous" (gdata = grouped_layout), "masked" (A [G][max_m][K],
    gdata = masked_m).  C float32 with D's shape."""
    A, SA, B, SB, C = _u8(A), _f32(SA), _u8(B), _f32(SB), _f32(C)
    K = A.shape[-1]
    N = B.shape[-2]
    k = {"dense": 0, "contiguous": 1, "masked": 2}[kind]
    G = 1 if B.ndim == 2 else B.shape[0]
    rows = A.shape[1] if kind == "masked" else A.shape[0]
    assert D.dtype == np.uint16 and D.flags["C_CONTIGUOUS"] and C.shape == D.shape
    gd = _i32(gdata if gdata is not None else np.zeros(1, np.int32))
    _check(_load().fp8bs_oracle_with_addend(k, _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(gd),
                                            _ptr(C), _ptr(D), G, rows, N, K))
    return D


def dense_layout(ab, A, SA, B, SB, C=None):
    """D (BF16 bits, [M][N]) for the stored forms ab in {"nt", "nn", "tn", "tt"}:
    A is [M][K] ("n" first) or [K][M] ("t"), B is [N][K] ("t" second) or [K][N] ("n").
    SA [M][K/128] and SB [ceil(N/128)][K/128] as in ``dense``; C float32 [M][N] or None."""
    assert ab in ("nt", "nn", "tn", "tt")
    A, SA, B, SB = _u8(A), _f32(SA), _u8(B), _f32(SB)
    a_t, b_t = ab[0] == "t", ab[1] == "t"
    M, K = (A.shape[1], A.shape[0]) if a_t else A.shape
    N = B.shape[0] if b_t else B.shape[1]
    assert (B.shape[1] if b_t else B.shape[0]) == K, "A and B disagree on K"
    D = np.zeros((M, N), dtype=np.uint16)
    Cp = None
    if C is not None:
        C = _f32(C)
        assert C.shape == (M, N)
        Cp = _ptr(C)
    _check(_load().fp8bs_oracle_dense_layout(int(a_t), int(b_t), _ptr(A), _ptr(SA), _ptr(B),
                                             _ptr(SB), Cp, _ptr(D), M, N, K))
    return D


def k_grouped(A, SA, B, SB, ks, C=None):
    """K-grouped product: A uint8 [K_total][M], B uint8 [K_total][N], SA float32
    [M][K_total/128], SB float32 [N][K_total/128], ks the G group sizes along K (each a
    multiple of 128, summing to K_total), C float32 [G][M][N] or None.  Returns FP32 D
    [G][M][N]."""
    A, SA, B, SB = _u8(A), _f32(SA), _u8(B), _f32(SB)
    ks = np.ascontiguousarray(ks, dtype=np.int64)
    K_total, M = A.shape
    N = B.shape[1]
    assert B.shape[0] == K_total
    G = ks.shape[0]
    D = np.zeros((G, M, N), dtype=np.float32)
    Cp = None
    if C is not None:
        C = _f32(C)
        assert C.shape == (G, M, N)
        Cp = _ptr(C)
    rc = _load().fp8bs_oracle_k_grouped(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(ks), Cp,
                                        _ptr(D), G, M, N, K_total)
    if rc != 0:
        raise ValueError("oracle rejected the group sizes (multiples of 128 summing to K_total)")
    return D

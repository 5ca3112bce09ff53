"""Shared helpers for the GPU parity tests: device copies, oracle runs, comparisons."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth

SENTINEL = 0x7FC1                 # a BF16 NaN payload the hardware conversion never produces
NORM_DIFF_MAX = 1e-4
REL_TOL = 2.0 ** -7
RMS_TOL = 1e-3


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def out_shape(p: synth.Problem):
    if p.kind == "masked":
        return (p.G, p.max_m, p.N)
    return (p.M, p.N)


def valid_row_mask(p: synth.Problem) -> np.ndarray:
    """Boolean mask over D's rows (flattened for masked) of rows the oracle writes."""
    if p.kind == "dense":
        return np.ones(p.M, bool)
    if p.kind == "contiguous":
        return (p.layout >= 0) & (p.layout < p.G)
    v = np.clip(p.masked_m, 0, p.max_m)
    return (np.arange(p.max_m)[None, :] < v[:, None]).reshape(-1)


def row_groups(p: synth.Problem) -> np.ndarray:
    """Group index of every D row (flattened), -1 where invalid."""
    if p.kind == "dense":
        return np.zeros(p.M, np.int64)
    if p.kind == "contiguous":
        g = p.layout.astype(np.int64)
        g[(g < 0) | (g >= p.G)] = -1
        return g
    g = np.repeat(np.arange(p.G), p.max_m)
    return np.where(valid_row_mask(p), g, -1)


class DeviceProblem:
    def __init__(self, p: synth.Problem, device="cuda"):
        self.p = p
        self.a = torch.from_numpy(p.A).to(device)
        self.sfa = fp8bs.sfa_mn_major(torch.from_numpy(p.SA)).to(device)
        b = p.B if p.kind != "dense" else p.B[0]
        self.b = torch.from_numpy(np.ascontiguousarray(b)).to(device)
        sb = p.SB if p.kind != "dense" else p.SB[0]
        self.sfb = torch.from_numpy(np.ascontiguousarray(sb)).to(device)
        self.layout = torch.from_numpy(p.layout).to(device) if p.layout is not None else None
        self.masked_m = torch.from_numpy(p.masked_m).to(device) if p.masked_m is not None else None
        self.d = torch.empty(out_shape(p), dtype=torch.int16, device=device)
        self.reset()

    def reset(self):
        self.d.fill_(SENTINEL)          # 0x7FC1 fits in int16

    def run(self, stream=None, workspace=True):
        """One call through the C ABI: the workspace (split-K capable) entry point by
        default, the workspace-free one with workspace=False."""
        p = self.p
        if p.kind == "dense":
            if workspace:
                fp8bs.fp8bs_dense_nt_ws(self.a, self.sfa, self.b, self.sfb, self.d, stream=stream)
            else:
                fp8bs.fp8bs_dense_nt(self.a, self.sfa, self.b, self.sfb, self.d, stream=stream)
        elif p.kind == "contiguous":
            f = fp8bs.fp8bs_grouped_contiguous_nt_ws if workspace else fp8bs.fp8bs_grouped_contiguous_nt
            f(self.a, self.sfa, self.b, self.sfb, self.d, self.layout, stream=stream)
        else:
            f = fp8bs.fp8bs_grouped_masked_nt_ws if workspace else fp8bs.fp8bs_grouped_masked_nt
            f(self.a, self.sfa, self.b, self.sfb, self.d, self.masked_m, expected_m=p.expected_m,
              stream=stream)

    def result(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.d.cpu().numpy().view(np.uint16)


def oracle_full(p: synth.Problem) -> np.ndarray:
    D = np.full(out_shape(p), SENTINEL, np.uint16)
    if p.kind == "dense":
        oracle.dense(p.A, p.SA, p.B[0], p.SB[0], D)
    elif p.kind == "contiguous":
        oracle.contiguous(p.A, p.SA, p.B, p.SB, p.layout, D)
    else:
        oracle.masked(p.A, p.SA, p.B, p.SB, p.masked_m, D)
    return D


def check_values(gpu_bits: np.ndarray, ref_bits: np.ndarray, what=""):
    """The floating-point bar: normalized diff and per-element bound."""
    x = bf16_bits_to_f64(gpu_bits.ravel())
    y = bf16_bits_to_f64(ref_bits.ravel())
    assert np.all(np.isfinite(y)), f"{what}: oracle produced non-finite values"
    assert np.all(np.isfinite(x)), f"{what}: GPU produced non-finite values at valid outputs"
    den = float((x * x).sum() + (y * y).sum())
    diff = 0.0 if den == 0.0 else 1.0 - 2.0 * float((x * y).sum()) / den
    assert diff <= NORM_DIFF_MAX, f"{what}: normalized diff {diff:.3e} > {NORM_DIFF_MAX}"
    rms = float(np.sqrt((y * y).mean())) if y.size else 0.0
    err = np.abs(x - y)
    bound = REL_TOL * np.abs(y) + RMS_TOL * rms
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{what}: {bad.size} outputs outside |gpu-ref| <= 2^-7|ref| + 1e-3 rms; "
                           f"first at flat index {bad[0]}: gpu {x[bad[0]]} ref {y[bad[0]]}")
    return diff


def check_full(p: synth.Problem, gpu: np.ndarray, ref: np.ndarray, what=""):
    """Whole-output comparison: valid rows to tolerance, the rest bit-exact sentinel."""
    rows = valid_row_mask(p)
    g2 = gpu.reshape(-1, p.N)
    r2 = ref.reshape(-1, p.N)
    assert np.all(r2[~rows] == SENTINEL)
    untouched = g2[~rows]
    assert np.all(untouched == SENTINEL), f"{what}: {int((untouched != SENTINEL).sum())} " \
                                          f"outputs written in rows that must stay untouched"
    return check_values(g2[rows], r2[rows], what)


def sample_points(p: synth.Problem, n_points: int, seed: int):
    """Valid (flat row, col) points, always including the first/last valid row and column."""
    rng = np.random.default_rng(seed)
    valid = np.nonzero(valid_row_mask(p))[0]
    rows = rng.choice(valid, size=n_points)
    cols = rng.integers(0, p.N, size=n_points)
    edge_r = np.array([valid[0], valid[-1], valid[0], valid[-1]])
    edge_c = np.array([0, p.N - 1, p.N - 1, 0])
    return np.concatenate([rows, edge_r]), np.concatenate([cols, edge_c])


def check_sampled(p: synth.Problem, gpu: np.ndarray, n_points=4096, seed=0, what=""):
    """Full-size check: every invalid row untouched (bit-exact), every valid output
    finite, and sampled outputs against the oracle computed one by one."""
    rows_ok = valid_row_mask(p)
    g2 = gpu.reshape(-1, p.N)
    untouched = g2[~rows_ok]
    assert np.all(untouched == SENTINEL), f"{what}: writes in rows that must stay untouched"
    vals = g2[rows_ok]
    assert not np.any((vals & 0x7F80) == 0x7F80), f"{what}: non-finite value in a valid row"
    r, c = sample_points(p, n_points, seed)
    grp = row_groups(p)[r]
    B = p.B if p.kind != "dense" else p.B[0]
    SB = p.SB if p.kind != "dense" else p.SB[0]
    _, ref = oracle.points(p.A.reshape(-1, p.K), p.SA.reshape(-1, p.K // 128), B, SB, r, grp, c)
    return check_values(g2[r, c], ref, what)

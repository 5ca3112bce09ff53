"""GPU parity of the K-grouped (MoE weight-gradient) GEMM against the oracle: every
instance compiled for it, empty groups, split-K with empty splits, the FP32 addend (also
in place), refusals, and the full-size workload on sampled features.

FP32 output bar.  The GPU sums each 128-K chunk in the matrix core, scales it with two
FP32 multiplies, adds it into an FP32 accumulator and finally adds C.  The matrix
core's FP8 chunk sum is not a correctly rounded FP32 sum: it drops low-order bits of
the products relative to the largest one (measured on MI355X over a million chunk
sums of normal, arbitrary, one-large-many-small and cancelling products: error at
most 2^-10.7 of the chunk's largest |a_k b_k|).  So with u = 2^-24,
E = sum_c |sa_c sb_c| max_k |a_k b_k| and T = |C| + sum_c |sa_c sb_c| sum_k |a_k b_k|,
the bar is

    |gpu - ref| <= 2^-8 E + (chunks + 4) u T + u |ref|

(the chunk sums with a 6x margin over the worst measured, the FP32 scaling and
accumulation of that many terms, and the oracle's single rounding), plus a normalized
difference of at most 1e-7.  E and T come from the decoded operands in float64."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
MN_INSTANCES = [i["instance"] for i in fp8bs.instances() if i["mn"]]


@pytest.fixture(autouse=True)
def _planner_choice():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)


def _dec(b):
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bound_terms(p, C):
    """(E, T, largest chunk count) of the module docstring, per output."""
    Aa = np.abs(_dec(p.A))
    Ba = np.abs(_dec(p.B))
    T = np.zeros((p.G, p.M, p.N))
    E = np.zeros((p.G, p.M, p.N))
    k0 = 0
    for g, kg in enumerate(p.ks):
        for c in range(k0 // 128, (k0 + int(kg)) // 128):
            a, b = Aa[128 * c:128 * c + 128], Ba[128 * c:128 * c + 128]
            s = np.abs(p.SA[:, c].astype(np.float64))[:, None] * \
                np.abs(p.SB[:, c].astype(np.float64))[None, :]
            T[g] += (a.T @ b) * s
            E[g] += (a[:, :, None] * b[:, None, :]).max(axis=0) * s
        k0 += int(kg)
    if C is not None:
        T += np.abs(C.astype(np.float64))
    return E, T, int((p.ks // 128).max()) if p.ks.size else 0


def _check(gpu, ref, p, C, what):
    E, T, chunks = _bound_terms(p, C)
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    bound = 2.0 ** -8 * E + (chunks + 4) * U * T + U * np.abs(r)
    err = np.abs(g - r)
    bad = np.nonzero(err > bound)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} outputs outside the bound; first "
                              f"{tuple(int(x[0]) for x in bad)}: gpu {g[bad][0]} ref {r[bad][0]}")
    den = float((g * g).sum() + (r * r).sum())
    if den > 0:
        assert 1.0 - 2.0 * float((g * r).sum()) / den <= 1e-7, what


def _device(p):
    a = torch.from_numpy(p.A).cuda()
    b = torch.from_numpy(p.B).cuda()
    sfa = fp8bs.sfa_mn_major(torch.from_numpy(p.SA)).cuda()
    sfb = fp8bs.sfa_mn_major(torch.from_numpy(p.SB)).cuda()
    return a, sfa, b, sfb


def _run(p, C=None, workspace=None, in_place=False):
    a, sfa, b, sfb = _device(p)
    d = torch.full((p.G, p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    c = None
    if C is not None:
        c = torch.from_numpy(C).cuda()
        if in_place:
            d.copy_(c)
            c = d
    fp8bs.fp8bs_k_grouped_tn_contiguous(a, sfa, b, sfb, d, list(p.ks), c=c, workspace=workspace)
    torch.cuda.synchronize()
    return d.cpu().numpy()


def _full(p, what, C=None, workspace=None, in_place=False):
    print(f"[gpu] k-grouped {what}: G={p.G} M={p.M} N={p.N} ks={list(p.ks)}", flush=True)
    gpu = _run(p, C, workspace, in_place)
    ref = oracle.k_grouped(p.A, p.SA, p.B, p.SB, p.ks, C)
    _check(gpu, ref, p, C, what)


@pytest.mark.parametrize("inst", MN_INSTANCES)
def test_every_instance(inst):
    fp8bs.force_instance(inst)
    # an empty group, a one-chunk group and a partly padded one; M, N ragged vs every tile
    p = synth.make_k_grouped(3, 80, 208, seed=900 + inst, counts=[0, 100, 300])
    _full(p, f"inst {inst}")


def test_planner_with_addend_and_in_place():
    p = synth.make_k_grouped(4, 128, 272, seed=910, total_tokens=900)
    C = (np.random.default_rng(911).standard_normal((4, 128, 272)) * 5).astype(np.float32)
    _full(p, "addend", C=C)
    _full(p, "addend in place", C=C, in_place=True)


@pytest.mark.parametrize("splits", [2, 5])
def test_split_k_with_empty_splits(splits):
    # group 0 has 1 chunk, fewer than the splits: its other splits are empty units
    p = synth.make_k_grouped(3, 96, 160, seed=920 + splits, counts=[128, 640, 0])
    C = np.random.default_rng(921).standard_normal((3, 96, 160)).astype(np.float32)
    fp8bs.force_splits(splits)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    _full(p, f"{splits} splits", C=C, workspace=ws)
    _full(p, f"{splits} splits, no addend", workspace=ws)


def test_all_groups_empty_gives_c_or_zero():
    p = synth.make_k_grouped(2, 32, 48, seed=930, counts=[0, 0])
    assert p.K == 0
    C = np.random.default_rng(931).standard_normal((2, 32, 48)).astype(np.float32)
    assert np.array_equal(_run(p, C), C)
    assert np.all(_run(p) == 0.0)


def test_constant_operands_bit_exact():
    ks = [256, 0, 384, 128]
    M, N = 48, 64
    K = sum(ks)
    p = synth.make_k_grouped(4, M, N, seed=940, counts=ks)
    p.A[:] = 0x40                                       # 2
    p.B[:] = 0xB0                                       # -0.5
    p.SA[:] = 0.125
    p.SB[:] = 4.0
    gpu = _run(p)
    for g, k in enumerate(ks):
        assert np.all(gpu[g] == np.float32(-k * 0.5)), g


def test_refusals():
    p = synth.make_k_grouped(2, 32, 48, seed=950, counts=[128, 128])
    a, sfa, b, sfb = _device(p)
    d = torch.zeros((2, 32, 48), dtype=torch.float32, device="cuda")
    with pytest.raises(fp8bs.FP8BSError):               # not multiples of 128
        fp8bs.fp8bs_k_grouped_tn_contiguous(a, sfa, b, sfb, d, [100, 156])
    with pytest.raises(fp8bs.FP8BSError):               # do not add up to k_total
        fp8bs.fp8bs_k_grouped_tn_contiguous(a, sfa, b, sfb, d, [128, 0])
    torch.cuda.synchronize()


@pytest.mark.parametrize("desc", synth.workload_shapes(5), ids=lambda d: d["name"])
def test_full_size_sampled_features(desc):
    """The benchmark's workload at full size, planner's launch: all outputs finite, and
    64 x 64 sampled (row, column) features of every group against the oracle."""
    p = synth.make(desc)
    print(f"[gpu] k-grouped full size {desc['name']}", flush=True)
    a, sfa, b, sfb = _device(p)
    d = torch.full((p.G, p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    ws_bytes = fp8bs.workspace_size(fp8bs.LAYOUT_K_GROUPED, p.M, p.N, p.K, p.G)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    fp8bs.fp8bs_k_grouped_tn_contiguous(a, sfa, b, sfb, d, list(p.ks), workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(d).all())
    rng = np.random.default_rng(p.seed)
    rows = np.unique(np.concatenate([rng.choice(p.M, 62, replace=False), [0, p.M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(p.N, 62, replace=False), [0, p.N - 1]]))
    sub = synth.KGroupedProblem(rows.size, cols.size, p.G, np.ascontiguousarray(p.A[:, rows]),
                                np.ascontiguousarray(p.SA[rows]),
                                np.ascontiguousarray(p.B[:, cols]),
                                np.ascontiguousarray(p.SB[cols]), p.ks, p.counts)
    ref = oracle.k_grouped(sub.A, sub.SA, sub.B, sub.SB, sub.ks)
    gpu = d.cpu().numpy()[:, rows][:, :, cols]
    _check(gpu, ref, sub, None, desc["name"])


def test_chunk_sum_precision_assumption():
    """One group of one chunk with unit scales: D is the matrix core's FP8 chunk sum
    itself.  Checks the measured property the bar above relies on -- error at most 2^-9
    of the largest |a_k b_k| -- on arbitrary codes, one large product with many small
    ones of one sign, and a cancelling large pair with small ones."""
    rng = np.random.default_rng(960)
    M, N = 192, 64
    A = rng.integers(0, 256, size=(128, M), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x7E
    B = rng.integers(0, 256, size=(128, N), dtype=np.uint8)
    B[(B & 0x7F) == 0x7F] = 0x7E
    B[:, N // 2:] = 0x38                                  # half the columns: b = 1
    for m in range(64, M):                                # one big (+ cancelling) + small
        e = (m - 64) % 12
        small = np.array([float(v) for v in (2.0 ** -e) * (1 + rng.integers(0, 8, 128) / 8)])
        codes = torch.from_numpy(small.astype(np.float32)).to(torch.float8_e4m3fn)
        A[:, m] = codes.view(torch.uint8).numpy()
        A[0, m] = 0x7E
        if m >= 128:
            A[1, m] = 0xFE
    p = synth.KGroupedProblem(M, N, 1, A, np.ones((M, 1), np.float32), B,
                              np.ones((N, 1), np.float32), np.array([128]), np.array([128]))
    gpu = _run(p)[0].astype(np.float64)
    prods = _dec(A)[:, :, None] * _dec(B)[:, None, :]
    exact = prods.sum(axis=0)
    largest = np.abs(prods).max(axis=0)
    ratio = np.abs(gpu - exact)[largest > 0] / largest[largest > 0]
    print(f"[gpu] chunk sum: max error / largest product = 2^{np.log2(ratio.max() + 1e-300):.1f}")
    assert ratio.max() <= 2.0 ** -9


def test_most_groups_the_call_takes():
    """256 groups (the most one call takes), many of them empty, the rest one or two
    chunks, with C: every group's offset in the kernel arguments is exercised."""
    rng = np.random.default_rng(970)
    counts = rng.integers(0, 200, size=256) * (rng.random(256) < 0.5)
    p = synth.make_k_grouped(256, 32, 48, seed=971, counts=counts)
    C = rng.standard_normal((256, 32, 48)).astype(np.float32)
    _full(p, "256 groups", C=C)


E8_MN_INSTANCES = [i["instance"] for i in fp8bs.instances() if i["mn"] and i["ue8m0"]]


def _run_e8(p, C=None, workspace=None):
    a = torch.from_numpy(p.A).cuda()
    b = torch.from_numpy(p.B).cuda()
    sfa = fp8bs.sfa_ue8m0_mn_major(torch.from_numpy(p.SA)).cuda()
    sfb = fp8bs.sfa_ue8m0_mn_major(torch.from_numpy(p.SB)).cuda()
    d = torch.full((p.G, p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    c = torch.from_numpy(C).cuda() if C is not None else None
    fp8bs.fp8bs_k_grouped_tn_contiguous_ue8m0(a, sfa, b, sfb, d, list(p.ks), c=c,
                                              workspace=workspace)
    torch.cuda.synchronize()
    return d.cpu().numpy()


def _full_e8(p, what, C=None, workspace=None):
    print(f"[gpu] k-grouped ue8m0 {what}: G={p.G} M={p.M} N={p.N} ks={list(p.ks)}", flush=True)
    gpu = _run_e8(p, C, workspace)
    _check(gpu, oracle.k_grouped(p.A, p.SA, p.B, p.SB, p.ks, C), p, C, what)


@pytest.mark.parametrize("inst", E8_MN_INSTANCES)
def test_ue8m0_every_instance(inst):
    """Power-of-two scales as packed E8M0 exponents: per-row A and per-column B exponents
    applied by the matrix core, no promotion step.  K = 5 chunks in one group, so a packed
    word is partly used and a group starts inside a word."""
    fp8bs.force_instance(inst)
    p = synth.make_k_grouped(3, 80, 208, seed=990 + inst, counts=[100, 0, 600], pow2=True)
    _full_e8(p, f"inst {inst}")


def test_ue8m0_planner_split_k_and_addend():
    p = synth.make_k_grouped(4, 96, 160, seed=995, counts=[128, 700, 0, 300], pow2=True)
    C = np.random.default_rng(996).standard_normal((4, 96, 160)).astype(np.float32)
    _full_e8(p, "planner, addend", C=C)
    fp8bs.force_splits(3)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    _full_e8(p, "3 splits, addend", C=C, workspace=ws)


def test_ue8m0_constant_operands_bit_exact():
    ks = [256, 0, 384, 128]
    p = synth.make_k_grouped(4, 48, 64, seed=997, counts=ks, pow2=True)
    p.A[:] = 0x40
    p.B[:] = 0xB0
    p.SA[:] = 0.125
    p.SB[:] = 4.0
    gpu = _run_e8(p)
    for g, k in enumerate(ks):
        assert np.all(gpu[g] == np.float32(-k * 0.5)), g

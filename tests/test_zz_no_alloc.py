"""The no-allocation dense entry point (fp8bs_dense_nt_noalloc), called through the C ABI:
same results as fp8bs_dense_nt_ws on the same inputs (bit for bit when both run the same
plan, which they do whenever the preferred plan's partial tiles fit the library's scratch
array), valid against the oracle, on two calls in a row with the second one smaller, so
that the second reads an array still holding the first call's partials."""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import SENTINEL, check_full, oracle_full

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _planner_choice():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)


def _device(p):
    a = torch.from_numpy(p.A).cuda()
    sfa = fp8bs.sfa_mn_major(torch.from_numpy(p.SA)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(p.B[0])).cuda()
    sfb = torch.from_numpy(np.ascontiguousarray(p.SB[0])).cuda()
    return a, sfa, b, sfb


def _out(p):
    return torch.full((p.M, p.N), SENTINEL, dtype=torch.int16, device="cuda")


# (M, N, K): a decode shape the planner splits, the pages' M=128 shape (split), then smaller
# ragged shapes, one of them unsplit
SEQUENCES = [
    [(64, 7168, 7168), (37, 1000, 1024)],
    [(128, 2112, 7168), (64, 2112, 2048)],
    [(256, 7168, 2048), (200, 300, 512)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join("x".join(map(str, t)) for t in s))
def test_noalloc_matches_the_workspace_call(seq):
    cap = fp8bs.noalloc_scratch_bytes()
    assert cap == 32 << 20
    for j, (m, n, k) in enumerate(seq):
        p = synth.make_dense(m, n, k, seed=7100 + 10 * j + m, outlier_frac=0.01)
        a, sfa, b, sfb = _device(p)
        ws_bytes = fp8bs.workspace_size(fp8bs.LAYOUT_DENSE, m, n, k)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        d_ws, d_na = _out(p), _out(p)
        _say(f"[gpu] noalloc call {j}: M={m} N={n} K={k} (preferred workspace {ws_bytes} B, "
             f"{fp8bs.describe_config(fp8bs.LAYOUT_DENSE, m, n, k)})")
        fp8bs.fp8bs_dense_nt_ws(a, sfa, b, sfb, d_ws, workspace=ws)
        fp8bs.fp8bs_dense_nt_noalloc(a, sfa, b, sfb, d_na)
        torch.cuda.synchronize()
        g_ws = d_ws.cpu().numpy().view(np.uint16)
        g_na = d_na.cpu().numpy().view(np.uint16)
        ref = oracle_full(p)
        check_full(p, g_na, ref, f"noalloc call {j}")
        check_full(p, g_ws, ref, f"workspace call {j}")
        if ws_bytes <= cap:               # same plan on both sides: same kernels, same bits
            assert np.array_equal(g_na, g_ws), f"call {j}: noalloc differs from the _ws call"


def test_noalloc_empty_and_refused_requests():
    lib = fp8bs._load()
    # m == 0: OK without launching or looking at a pointer; K not a multiple of 128: refused
    assert lib.fp8bs_dense_nt_noalloc(None, None, None, None, None, 0, 64, 128, None) == 0
    assert lib.fp8bs_dense_nt_noalloc(None, None, None, None, None, 64, 256, 100, None) == 1
    # a pinned split count whose partial tiles exceed the array is refused before launching
    big = synth.make_dense(4096, 2048, 2048, seed=7191)
    a, sfa, b, sfb = _device(big)
    d = _out(big)
    fp8bs.force_splits(16)
    with pytest.raises(fp8bs.FP8BSError) as e:
        fp8bs.fp8bs_dense_nt_noalloc(a, sfa, b, sfb, d)
    assert e.value.status == 3
    fp8bs.force_splits(0)
    torch.cuda.synchronize()
    assert np.all(d.cpu().numpy().view(np.uint16) == SENTINEL)   # nothing was written

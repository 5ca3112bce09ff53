"""HIP graph capture of the entry points, the decode-time use the pages describe for the
masked layout (the host cannot read the per-expert counts, so the kernel reads them on the
device): each call is captured once and the graph is replayed several times, with eager
work between replays (new device-side masks or group indices, output reset), and every
replay is checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import DeviceProblem, check_full, oracle_full
import test_gpu_kgrouped as kg

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _planner_choice():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_masked_graph_replays_follow_the_device_mask():
    p = synth.make_masked(6, 128, 320, 512, seed=1100, masked_m=[0, 128, 5, 77, 128, 1])
    dp = DeviceProblem(p)
    ws = torch.empty(32 << 20, dtype=torch.uint8, device="cuda")
    g = _capture(lambda: fp8bs.fp8bs_grouped_masked_nt_ws(dp.a, dp.sfa, dp.b, dp.sfb, dp.d,
                                                          dp.masked_m, expected_m=64,
                                                          workspace=ws))
    rng = np.random.default_rng(1101)
    for r in range(4):
        p.masked_m = rng.integers(0, 129, size=6).astype(np.int32)
        print(f"[gpu] masked graph replay {r}: masked_m {list(p.masked_m)}", flush=True)
        dp.masked_m.copy_(torch.from_numpy(p.masked_m))   # eager, outside the graph
        dp.reset()
        g.replay()
        check_full(p, dp.result(), oracle_full(p), f"masked graph replay {r}")


def test_contiguous_graph_replays_follow_the_device_layout():
    p = synth.make_contiguous(4, 256, 384, seed=1110, counts=[100, 300, 0, 60])
    dp = DeviceProblem(p)
    g = _capture(lambda: fp8bs.fp8bs_grouped_contiguous_nt(dp.a, dp.sfa, dp.b, dp.sfb, dp.d,
                                                           dp.layout))
    # new row-to-expert maps over the same 640 rows, written on the device between replays
    for r, counts in enumerate([[10, 130, 120, 1], [0, 512, 0, 100], [640, 0, 0, 0],
                                [0, 0, 0, 0]]):
        lay = synth.contiguous_layout(counts)
        p.layout = np.concatenate([lay, np.full(p.M - lay.size, -1, np.int32)])
        print(f"[gpu] contiguous graph replay {r}: counts {counts}", flush=True)
        dp.layout.copy_(torch.from_numpy(p.layout))
        dp.reset()
        g.replay()
        check_full(p, dp.result(), oracle_full(p), f"contiguous graph replay {r}")


def test_split_k_graph_replays_are_bit_identical():
    p = synth.make_dense(64, 2112, 2048, seed=1120)
    dp = DeviceProblem(p)
    fp8bs.force_splits(4)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    g = _capture(lambda: fp8bs.fp8bs_dense_nt_ws(dp.a, dp.sfa, dp.b, dp.sfb, dp.d, workspace=ws))
    ref = oracle_full(p)
    first = None
    for r in range(3):
        print(f"[gpu] split-K graph replay {r}", flush=True)
        ws.fill_(0xFF)                                  # stale partials must not leak in
        dp.reset()
        g.replay()
        got = dp.result()
        check_full(p, got, ref, f"split-K graph replay {r}")
        if first is None:
            first = got.copy()
        assert np.array_equal(got, first)


def test_k_grouped_graph_replays():
    """The group sizes along K are host values, fixed at capture: every replay recomputes
    the same result into an output poisoned with NaN between replays."""
    p = synth.make_k_grouped(3, 64, 96, seed=1130, counts=[200, 0, 130])
    a, sfa, b, sfb = kg._device(p)
    d = torch.empty((3, 64, 96), dtype=torch.float32, device="cuda")
    g = _capture(lambda: fp8bs.fp8bs_k_grouped_tn_contiguous(a, sfa, b, sfb, d, list(p.ks)))
    ref = oracle.k_grouped(p.A, p.SA, p.B, p.SB, p.ks)
    first = None
    for r in range(3):
        print(f"[gpu] k-grouped graph replay {r}", flush=True)
        d.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = d.cpu().numpy()
        kg._check(got, ref, p, None, f"k-grouped graph replay {r}")
        if first is None:
            first = got.copy()
        assert np.array_equal(got, first)
